// Block router: mean pooling of Q and K per block, pair scores with the soft
// geometric bias, and top-K selection into ascending CSR lists.
//
// [Velox: Spatial Memory Makes World Models Efficient -- Methodology, Step 4:
//  each layer scores the KV blocks a query block can see with the block
//  averages of its queries and keys; overlaps above tau, rescaled to g_hat,
//  scale that distribution by (1 + lambda g_hat) before it is normalised
//  again (a boost of at most 1 + lambda); Key Contributions 2: where the
//  geometry covers nothing the model's own scores decide; Methodology,
//  Step 5: each row keeps its highest-scoring blocks, up to a budget]
//
// Arithmetic is float64 throughout.  A block mean is the exact sum of its
// valid rows (for a column whose nonzero magnitudes span less than 2^39 in
// bf16, or 2^74 in float32: exact_sum.h), rounded once and divided once, so
// it does not depend on summation order.  The fused distribution softmax(s) * (1 + lambda g_hat) / Z orders
// a row exactly as kappa = s + log1p(lambda g_hat) does (Z is a positive
// per-row constant, log is increasing), so kappa is what gets ranked; a row
// whose overlap is all zero has g_hat = 0 everywhere and so keeps kappa = s,
// the unbiased route.  Ranking is the total order (kappa descending, block
// index ascending).
#include <hip/hip_runtime.h>

#include <mutex>

#include "exact_sum.h"
#include "kernels.h"

// Fixed device scratch of bsa_route_topk_static (callers that cannot
// allocate): one copy per GPU, held from the library's load to the end of
// the process.  Host code never passes `scratch` itself to a kernel (in host
// code the name is a host-side stand-in, not a device address); it uses the
// address hipGetSymbolAddress returns on each device.
static __device__ __align__(256) unsigned char scratch[BSA_ROUTE_STATIC_SCRATCH_BYTES];

namespace bsa {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ double bf16_to_f64(uint32_t bits16) {
    return (double)__uint_as_float(bits16 << 16);
}

// Mean of the valid rows of each block: one workgroup of 4 waves per block,
// grid = (blocks, heads).  Wave w sums rows w, w + 4, ... of its quarter of
// the block; lane l owns one 16-byte chunk (l % chunks) of rows l / chunks,
// + groups, ...  Sums are exact (exact_sum.h), combined over the row groups
// with butterfly shuffles and over the four waves through LDS; the order
// does not change the result.  Four waves per block keep
// enough loads in flight when only a chunk's worth of blocks is pooled.
template <bool BF16>
__global__ void __launch_bounds__(kThreads)
pool_kernel(const void* __restrict__ x, int64_t head_stride, int d, int block,
            const int32_t* __restrict__ lens, int b_begin, int nb, double* __restrict__ out,
            int64_t out_head_blocks) {
    constexpr int CE = BF16 ? 8 : 4;  // elements per 16-byte chunk
    constexpr int NW = kThreads / 64;
    __shared__ double part_hi[NW][128], part_lo[NW][128];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int b = b_begin + blockIdx.x, h = blockIdx.y;
    int valid = lens ? lens[b] : block;
    valid = valid < 0 ? 0 : (valid > block ? block : valid);
    const int chunks = d / CE, groups = 64 / chunks;
    const int ch = lane % chunks, g = lane / chunks;
    Acc<BF16> acc[CE];
    const int64_t base = h * head_stride + (int64_t)b * block * d + ch * CE;
#pragma unroll 8
    for (int row = w * groups + g; row < valid; row += NW * groups) {
        if (BF16) {
            const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + base + (int64_t)row * d);
            const uint32_t wd[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc[2 * e].add(bf16_to_f64(wd[e] & 0xFFFFu));
                acc[2 * e + 1].add(bf16_to_f64(wd[e] >> 16));
            }
        } else {
            const float4 f = *reinterpret_cast<const float4*>(static_cast<const float*>(x) + base + (int64_t)row * d);
            acc[0].add((double)f.x);
            acc[1].add((double)f.y);
            acc[2].add((double)f.z);
            acc[3].add((double)f.w);
        }
    }
    for (int off = chunks; off < 64; off <<= 1)
#pragma unroll
        for (int e = 0; e < CE; ++e) acc[e].add(acc[e].shfl_xor(off));
    if (g == 0)
#pragma unroll
        for (int e = 0; e < CE; ++e) {
            part_hi[w][ch * CE + e] = acc[e].hi();
            part_lo[w][ch * CE + e] = acc[e].lo();
        }
    __syncthreads();
    const int t = threadIdx.x;
    if (t < d) {
        Acc<BF16> sum = Acc<BF16>::make(part_hi[0][t], part_lo[0][t]);
#pragma unroll
        for (int u = 1; u < NW; ++u) sum.add(Acc<BF16>::make(part_hi[u][t], part_lo[u][t]));
        out[(h * out_head_blocks + b) * d + t] = valid > 0 ? sum.hi() / (double)valid : 0.0;
    }
}

// Which query-block rows of the overlap are all zero (flag bit 0) or never
// above tau (flag bit 1).  grid = nqb.
__global__ void __launch_bounds__(kThreads)
overlap_flags_kernel(const float* __restrict__ overlap, int64_t ors, int n_cand, double tau,
                     int32_t* __restrict__ flags) {
    __shared__ int any_nz[kThreads / 64], any_vet[kThreads / 64];
    const int i = blockIdx.x, t = threadIdx.x;
    int nz = 0, vet = 0;
    for (int j = t; j < n_cand; j += kThreads) {
        const float g = overlap[(int64_t)i * ors + j];
        nz |= g != 0.0f;
        vet |= ((double)g > tau) && g > 0.0f;
    }
    nz = __any(nz);
    vet = __any(vet);
    if ((t & 63) == 0) {
        any_nz[t >> 6] = nz;
        any_vet[t >> 6] = vet;
    }
    __syncthreads();
    if (t == 0) {
        int a = 0, v = 0;
        for (int w = 0; w < kThreads / 64; ++w) {
            a |= any_nz[w];
            v |= any_vet[w];
        }
        flags[i] = (a ? 0 : 1) | (v ? 0 : 2);
    }
}

// kappa[h][i][j] = (qbar_i . kbar_j) * scale + log1p(lambda * g_hat_ij).
// Selection keys with the float64 matrix cores.  A workgroup of 4 waves
// takes 32 candidates (two 16-candidate tiles) and 48 query blocks (three
// 16-row tiles) of one head; grid = (ceil(n_cand / 32), heads, ceil(nqb /
// 48)).  The channels are split among the waves: wave w takes the 16-channel
// steps w, w + 4, ..., so each wave loads all of its operands at once and
// the workgroup needs one memory round trip.  In a step, lane l (g = l / 16,
// r = l % 16) holds channels 4g .. 4g+3 of pooled key (candidate r of a
// tile) and pooled query (row r of a tile) as 32 contiguous bytes and feeds
// them to four v_mfma_f64_16x16x4f64, the i-th on channel 4g + i: over the
// lane groups that is a 16 x 16 x 4 product over channels 4g + i, so the
// four products cover the step (the same channel order on both operands).
// The four waves' partial products are summed through LDS in wave order.
constexpr int kScoreJ = 32, kScoreRows = 48, kScoreTiles = kScoreRows / 16, kScoreJT = kScoreJ / 16;
constexpr int kScoreMaxSteps = 2;  // 16-channel steps per wave (d <= 128)

typedef double f64x4 __attribute__((ext_vector_type(4)));

__device__ __attribute__((noinline)) double overlap_bias(double g, double lambda, double g_ref, double tau) {
    const double gh = g <= tau ? 0.0 : fmin(1.0, g / g_ref);
    return log1p(lambda * gh);
}

__device__ __forceinline__ f64x4 load_f64x4(const double* p) {
    const double2 a = *reinterpret_cast<const double2*>(p);
    const double2 b = *reinterpret_cast<const double2*>(p + 2);
    return f64x4{a.x, a.y, b.x, b.y};
}

__global__ void __launch_bounds__(kThreads)
score_kernel(const double* __restrict__ qbar, int64_t qbar_head_stride, const double* __restrict__ kbar,
             int64_t kbar_head_blocks,
             int nqb, int n_cand, int d, double scale, const float* __restrict__ overlap, int64_t ors,
             double lambda, double g_ref, double tau, const float* __restrict__ coverage, double eta_cov,
             double* __restrict__ keys) {
    __shared__ f64x4 part[kThreads / 64][kScoreJT * kScoreTiles][64];
    const int h = blockIdx.y, t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int g = lane >> 4, r = lane & 15;
    const int j0 = blockIdx.x * kScoreJ, r0 = blockIdx.z * kScoreRows;
    const int steps = d / 16;
    const f64x4 zero = {0.0, 0.0, 0.0, 0.0};
    f64x4 kb[kScoreMaxSteps][kScoreJT], qa[kScoreMaxSteps][kScoreTiles];
#pragma unroll
    for (int k = 0; k < kScoreMaxSteps; ++k) {
        const int st = w + 4 * k;
#pragma unroll
        for (int v = 0; v < kScoreJT; ++v) {
            const int jc = j0 + 16 * v + r;
            kb[k][v] = zero;
            if (st < steps && jc < n_cand)
                kb[k][v] = load_f64x4(kbar + ((int64_t)h * kbar_head_blocks + jc) * d + 16 * st + 4 * g);
        }
#pragma unroll
        for (int u = 0; u < kScoreTiles; ++u) {
            const int row = r0 + 16 * u + r;
            qa[k][u] = zero;
            if (st < steps && row < nqb)
                qa[k][u] = load_f64x4(qbar + h * qbar_head_stride + (int64_t)row * d + 16 * st + 4 * g);
        }
    }
    f64x4 acc[kScoreJT][kScoreTiles];
#pragma unroll
    for (int v = 0; v < kScoreJT; ++v)
#pragma unroll
        for (int u = 0; u < kScoreTiles; ++u) acc[v][u] = zero;
#pragma unroll
    for (int k = 0; k < kScoreMaxSteps; ++k)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int v = 0; v < kScoreJT; ++v)
#pragma unroll
                for (int u = 0; u < kScoreTiles; ++u)
                    acc[v][u] = __builtin_amdgcn_mfma_f64_16x16x4f64(qa[k][u][i], kb[k][v][i], acc[v][u], 0, 0, 0);
#pragma unroll
    for (int v = 0; v < kScoreJT; ++v)
#pragma unroll
        for (int u = 0; u < kScoreTiles; ++u) part[w][v * kScoreTiles + u][lane] = acc[v][u];
    __syncthreads();
    // each wave finishes the tiles v * kScoreTiles + u == w (mod 4): the sum
    // of the four waves' partials, in wave order.  Accumulator layout: lane
    // l, element e holds row l / 16 + 4e of the row tile and candidate
    // l % 16 of the candidate tile.
    for (int tile = w; tile < kScoreJT * kScoreTiles; tile += kThreads / 64) {
        const int v = tile / kScoreTiles, u = tile % kScoreTiles;
        f64x4 sum = part[0][tile][lane];
#pragma unroll
        for (int x = 1; x < kThreads / 64; ++x) sum += part[x][tile][lane];
        const int jc = j0 + 16 * v + r;
        if (jc >= n_cand) continue;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = r0 + 16 * u + g + 4 * e;
            if (i >= nqb) continue;
            double kap = sum[e] * scale;
            // the geometric bias applies to well-covered query blocks only
            // (all of them when no coverage is given)
            if (overlap && (!coverage || coverage[i] >= (float)eta_cov))
                kap += overlap_bias((double)overlap[(int64_t)i * ors + jc], lambda, g_ref, tau);
            keys[((int64_t)h * nqb + i) * n_cand + jc] = kap;
        }
    }
}

// Integer sums and scans over a 1024-thread workgroup: within each wave by
// shuffles, across the 16 waves through a 16-int LDS array (two barriers).
// Integer addition is exact, so the order does not matter.
__device__ __forceinline__ int block_sum_1024(int v, int* sh16) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    __syncthreads();  // sh16 free (the previous use has been read)
    if (lane == 0) sh16[w] = v;
    __syncthreads();
    int r = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) r += sh16[i];
    return r;
}

// Exclusive prefix sum of v over the workgroup's threads in thread order;
// *total receives the sum of all of them.
__device__ __forceinline__ int block_excl_scan_1024(int v, int* sh16, int* total) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    int incl = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int up = __shfl_up(incl, off);
        if (lane >= off) incl += up;
    }
    __syncthreads();  // sh16 free
    if (lane == 63) sh16[w] = incl;
    __syncthreads();
    int before = 0, all = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int x = sh16[i];
        before += i < w ? x : 0;
        all += x;
    }
    *total = all;
    return before + incl - v;
}

// Single workgroup: per-row list lengths, the exclusive prefix sum into
// row_ptr, and the fallback counts.
__global__ void __launch_bounds__(1024)
rowptr_kernel(int heads, int nqb, int nkb, int n_cand, int block, const int32_t* __restrict__ q_len,
              const int32_t* __restrict__ kv_len, int k_fixed, const int32_t* __restrict__ k_per_row,
              int k_max, const int32_t* __restrict__ flags, int32_t* __restrict__ row_ptr,
              int32_t* __restrict__ keff, int32_t* __restrict__ fallback_counts) {
    __shared__ int sh[16];
    const int t = threadIdx.x;
    int c_vis = 0, c_tail = 0;
    for (int j = t; j < nkb; j += 1024) {
        const int v = kv_len ? kv_len[j] : block;
        if (v > 0) {
            if (j < n_cand)
                ++c_vis;
            else
                ++c_tail;
        }
    }
    const int n_vis = block_sum_1024(c_vis, sh);
    const int n_tail = block_sum_1024(c_tail, sh);
    const int rows = heads * nqb;
    int carry = 0;
    for (int base = 0; base < rows; base += 1024) {
        const int r = base + t;
        int tot = 0;
        if (r < rows) {
            const int i = r % nqb;
            const int vq = q_len ? q_len[i] : block;
            int kr = k_fixed;
            if (k_per_row) {
                kr = k_per_row[r];
                kr = kr < 0 ? 0 : (kr > k_max ? k_max : kr);
            }
            const int ke = vq > 0 ? (kr < n_vis ? kr : n_vis) : 0;
            keff[r] = ke;
            tot = vq > 0 ? ke + n_tail : 0;
        }
        int chunk_total;
        const int excl = block_excl_scan_1024(tot, sh, &chunk_total);
        if (r < rows) row_ptr[r] = carry + excl;
        carry += chunk_total;
    }
    if (t == 0) row_ptr[rows] = carry;
    if (fallback_counts) {
        int z = 0, u = 0;
        if (flags) {
            for (int i = t; i < nqb; i += 1024) {
                z += flags[i] & 1;
                u += (flags[i] >> 1) & 1;
            }
        }
        z = block_sum_1024(z, sh);
        u = block_sum_1024(u, sh);
        if (t == 0) {
            fallback_counts[0] = z;
            fallback_counts[1] = u;
        }
    }
}

// Order-preserving map of a double to an unsigned integer (larger double,
// larger key); -0 and +0 map to the same key.  Every finite or infinite
// double maps above 0, so 0 marks "not a candidate".
__device__ __forceinline__ unsigned long long order_key(double v) {
    if (v == 0.0) v = 0.0;
    const long long b = __double_as_longlong(v);
    return b < 0 ? ~(unsigned long long)b : ((unsigned long long)b | 0x8000000000000000ull);
}

__device__ __forceinline__ unsigned long long shfl_xor_u64(unsigned long long v, int m) {
    const int lo = __shfl_xor((int)(unsigned)v, m), hi = __shfl_xor((int)(unsigned)(v >> 32), m);
    return ((unsigned long long)(unsigned)hi << 32) | (unsigned)lo;
}

// (key, index) order of the selection: larger key first, lower index first
// among equal keys.
__device__ __forceinline__ bool sel_before(unsigned long long ka, int ia, unsigned long long kb, int ib) {
    return ka > kb || (ka == kb && ia < ib);
}

// The k-th largest of 32-bit values held by a wave, N per lane, among
// those whose flag is set, by bisection on the bits: the largest t with at
// least k flagged values >= t, built from the most significant bit down (0
// when fewer than k values are flagged).  The count of each trial is a
// ballot, so the bound stays wave-uniform and nothing moves between lanes.
template <int N>
__device__ __forceinline__ uint32_t wave_kth_largest32(const uint32_t (&v)[N], const bool (&in)[N], int k) {
    uint32_t p = 0;
    k = __builtin_amdgcn_readfirstlane(k);  // the same for every lane; keeps the bound scalar
#pragma unroll
    for (int b = 31; b >= 0; --b) {
        const uint32_t t = p | (1u << b);
        int c = 0;
#pragma unroll
        for (int n = 0; n < N; ++n) c += __popcll(__ballot(in[n] && v[n] >= t));
        if (c >= k) p = t;
    }
    return p;
}

__device__ __forceinline__ uint32_t hi32(unsigned long long x) { return (uint32_t)(x >> 32); }

// Fast path of the top-ke threshold (see select_threshold) for ke <= 64 R:
// the R largest high words of each lane hold ke values that are high words
// of distinct keys, so the ke-th largest of them bounds the high word of
// the ke-th largest key from below.  The keys that reach the bound are
// gathered, G per lane (false when more than 64 G do), and the ke-th
// largest of them is found by bisection on the high words, then, only when
// several gathered keys share the deciding high word, on their low words.
// `ck` is a 64 G-entry per-wave LDS scratch.
template <int KPL, int R, int G>
__device__ __forceinline__ bool select_fast(const unsigned long long (&key)[KPL], int ke, int lane,
                                            unsigned long long* ck, unsigned long long& prefix, int& need,
                                            bool& all_eq) {
    const unsigned long long lt_mask = (1ull << lane) - 1ull;
    uint32_t top[R];
    bool lane_in[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        top[r] = 0;
        lane_in[r] = true;
    }
#pragma unroll
    for (int m = 0; m < KPL; ++m) {
        uint32_t x = hi32(key[m]);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const uint32_t hi = top[r] > x ? top[r] : x;
            x = top[r] > x ? x : top[r];
            top[r] = hi;
        }
    }
    const uint32_t lh = wave_kth_largest32<R>(top, lane_in, ke);
    int c = 0;
#pragma unroll
    for (int m = 0; m < KPL; ++m) {
        const bool cand = key[m] != 0 && hi32(key[m]) >= lh;
        const unsigned long long b = __ballot(cand);
        const int at = c + __popcll(b & lt_mask);
        if (cand && at < 64 * G) ck[at] = key[m];
        c += __popcll(b);
    }
    if (c > 64 * G) return false;
    __builtin_amdgcn_wave_barrier();
    __asm__ volatile("" ::: "memory");
    unsigned long long kv[G];
    uint32_t th[G];
    bool nz[G];
#pragma unroll
    for (int n = 0; n < G; ++n) {
        kv[n] = lane + 64 * n < c ? ck[lane + 64 * n] : 0ull;
        th[n] = hi32(kv[n]);
        nz[n] = kv[n] != 0;
    }
    const uint32_t ph = wave_kth_largest32<G>(th, nz, ke);
    int above = 0, tied = 0;
#pragma unroll
    for (int n = 0; n < G; ++n) {
        above += __popcll(__ballot(nz[n] && th[n] > ph));
        tied += __popcll(__ballot(nz[n] && th[n] == ph));
    }
    const int need_h = ke - above;  // 1 <= need_h <= tied
    uint32_t pl = 0;
    if (need_h < tied) {
        uint32_t tl[G];
        bool in_h[G];
#pragma unroll
        for (int n = 0; n < G; ++n) {
            tl[n] = (uint32_t)kv[n];
            in_h[n] = nz[n] && th[n] == ph;
        }
        pl = wave_kth_largest32<G>(tl, in_h, need_h);
    }
    prefix = ((unsigned long long)ph << 32) | pl;
    int gt = 0, eq = 0;
#pragma unroll
    for (int n = 0; n < G; ++n) {
        gt += __popcll(__ballot(kv[n] > prefix));
        eq += __popcll(__ballot(kv[n] == prefix));
    }
    need = ke - gt;
    all_eq = need == eq;
    __builtin_amdgcn_wave_barrier();
    __asm__ volatile("" ::: "memory");
    return true;
}

// Largest per-wave candidate scratch of the fast paths (entries).
constexpr int kSelScratch = 64 * 8;

// Threshold of the top-ke selection over the keys of one row held by a
// wave (lane l: keys of candidates l + 64 m; 0 = not a candidate): the
// selected set is every key > prefix plus the first `need` keys == prefix
// in ascending candidate order, which is the total order (key descending,
// index ascending); prefix is the ke-th largest key and need = ke minus the
// number of keys above it.  `all_eq` reports that every key equal to
// prefix is selected (then no ranking among equal keys is needed).  The
// fast path takes the lane top-2 bound for ke <= 64, top-4 for ke <= 128
// and top-8 for ke <= 256; when it does not apply (more candidates reach
// the bound than it gathers, or ke > 256), a radix select over 8-bit digits
// (most significant first, a 256-bin histogram per wave in LDS) finds the
// ke-th largest key and how many keys equal to it are needed.  `hist` is a
// 256-int and cand_key a kSelScratch-entry per-wave LDS scratch.
template <int KPL>
__device__ __forceinline__ void select_threshold(const unsigned long long (&key)[KPL], int ke, int lane,
                                                 int* hist, unsigned long long* cand_key,
                                                 unsigned long long& prefix, int& need, bool& all_eq) {
    unsigned long long mask = 0;
    bool found = false;
    if (ke > 0 && ke <= 64)
        found = select_fast<KPL, 2, 2>(key, ke, lane, cand_key, prefix, need, all_eq);
    else if (ke > 64 && ke <= 128)
        found = select_fast<KPL, 4, 4>(key, ke, lane, cand_key, prefix, need, all_eq);
    else if (ke > 128 && ke <= 256)
        found = select_fast<KPL, 8, 8>(key, ke, lane, cand_key, prefix, need, all_eq);
    if (!found) {
        prefix = 0;
        need = ke;
        all_eq = false;
    }
    if (ke > 0 && !found) {
#pragma unroll 1
        for (int shift = 56; shift >= 0; shift -= 8) {
#pragma unroll
            for (int b = 0; b < 4; ++b) hist[lane * 4 + b] = 0;
#pragma unroll
            for (int m = 0; m < KPL; ++m)
                if (key[m] != 0 && (key[m] & mask) == prefix) atomicAdd(&hist[(key[m] >> shift) & 255], 1);
            // lane l owns bins 255-4l .. 252-4l (descending); find the bin
            // where the count of keys from the top reaches `need`
            int c[4], tot = 0;
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                c[b] = hist[255 - 4 * lane - b];
                tot += c[b];
            }
            int incl = tot;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const int up = __shfl_up(incl, off);
                if (lane >= off) incl += up;
            }
            const unsigned long long reach = __ballot(incl >= need);
            const int owner = __ffsll((long long)reach) - 1;
            int digit = 0, above = 0;
            if (lane == owner) {
                int acc = incl - tot;  // keys in bins above this lane's first bin
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    if (acc + c[b] >= need) {
                        digit = 255 - 4 * lane - b;
                        above = acc;
                        break;
                    }
                    acc += c[b];
                }
            }
            digit = __shfl(digit, owner);
            above = __shfl(above, owner);
            need -= above;
            prefix |= (unsigned long long)digit << shift;
            mask |= 0xFFull << shift;
        }
    }
}

// Three waves per SIMD (at most 168 registers; the compiler fits every
// instance without spilling): one wave per row spends most of its time in
// short dependent ballot chains, so more rows in flight per SIMD is what
// shortens the launch (2960 rows of 3478 candidates, blocks of 64: 2 -> 3 waves per
// SIMD takes the router from 187 to 156 us, the same lists).
// One wave per (head, query block) row: the threshold of its top-K_eff,
// then the selected indices in ascending order (ballot prefix counts),
// followed by the dense tail.  grid = ceil(rows / 4), 4 waves per
// workgroup, no barriers.  The keys and the block lengths are loaded
// together, so a row costs one memory round trip before the selection.
template <int KPL>
__global__ void __launch_bounds__(kThreads, 3)
topk_kernel(const double* __restrict__ keys, int rows, int nqb, int n_cand, int nkb, int block,
            const int32_t* __restrict__ q_len, const int32_t* __restrict__ kv_len, int k_fused,
            int32_t* __restrict__ row_ptr, const int32_t* __restrict__ keff, int32_t* __restrict__ col_idx,
            int32_t* __restrict__ zero_counts) {
    __shared__ int hist_all[kThreads / 64][256];
    __shared__ unsigned long long cand_key[kThreads / 64][kSelScratch];
    // the wave index is the same for every lane: row, query block and budget stay scalar
    const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r = blockIdx.x * (kThreads / 64) + w;
    if (r >= rows) return;
    const int i = r % nqb;
    const int vq = q_len ? q_len[i] : block;
    const unsigned long long lt_mask = (1ull << lane) - 1ull;
    const double* row = keys + (int64_t)r * n_cand;
    // keys of the visible candidates (0: not a candidate)
    unsigned long long key[KPL];
    int n_vis = 0;
#pragma unroll
    for (int m = 0; m < KPL; ++m) {
        const int j = lane + 64 * m;
        double x = 0.0;
        int v = 0;
        if (j < n_cand) {
            x = row[j];
            v = kv_len ? kv_len[j] : block;
        }
        key[m] = v > 0 ? order_key(x) : 0ull;
        n_vis += __popcll(__ballot(key[m] != 0));
    }
    int start, ke;
    if (k_fused >= 0) {
        // fixed budget: every non-empty row has min(K, visible candidates)
        // + the visible tail blocks, so a row's start is a count of the
        // non-empty query blocks before it
        int n_tail = 0;
        for (int j0 = n_cand; j0 < nkb; j0 += 64) {
            const int jb = j0 + lane;
            n_tail += __popcll(__ballot(jb < nkb && (kv_len ? kv_len[jb] : block) > 0));
        }
        int before = 0, nonempty = 0;
        for (int i0 = 0; i0 < nqb; i0 += 64) {
            const int ib = i0 + lane;
            const bool ne = ib < nqb && (q_len ? q_len[ib] : block) > 0;
            nonempty += __popcll(__ballot(ne));
            before += __popcll(__ballot(ne && ib < i));
        }
        const int ke0 = k_fused < n_vis ? k_fused : n_vis;
        const int len = ke0 + n_tail;
        start = ((r / nqb) * nonempty + before) * len;
        ke = vq > 0 ? ke0 : 0;
        if (lane == 0) {
            row_ptr[r] = start;
            if (r == rows - 1) row_ptr[rows] = start + (vq > 0 ? len : 0);
            if (r == 0 && zero_counts) zero_counts[0] = zero_counts[1] = 0;
        }
    } else {
        if (vq <= 0) return;
        start = row_ptr[r];
        ke = keff[r];
    }
    if (vq <= 0) return;
    int* hist = hist_all[w];

    unsigned long long prefix;
    int need;
    bool all_eq;
    select_threshold<KPL>(key, ke, lane, hist, cand_key[w], prefix, need, all_eq);
    // ordered compaction: key > t, or key == t and among the first `need`
    // (every key >= t when all the equal keys are taken)
    int base = start;
    if (ke > 0 && all_eq) {
#pragma unroll
        for (int m = 0; m < KPL; ++m) {
            const bool sel = key[m] != 0 && key[m] >= prefix;
            const unsigned long long bs = __ballot(sel);
            if (sel) col_idx[base + __popcll(bs & lt_mask)] = lane + 64 * m;
            base += __popcll(bs);
        }
    } else {
        int eq_seen = 0;
#pragma unroll
        for (int m = 0; m < KPL; ++m) {
            const bool gt = ke > 0 && key[m] > prefix;
            const bool eq = ke > 0 && key[m] != 0 && key[m] == prefix;
            const unsigned long long beq = __ballot(eq);
            const int rank = eq_seen + __popcll(beq & lt_mask);
            eq_seen += __popcll(beq);
            const bool sel = gt || (eq && rank < need);
            const unsigned long long bs = __ballot(sel);
            if (sel) col_idx[base + __popcll(bs & lt_mask)] = lane + 64 * m;
            base += __popcll(bs);
        }
    }
    for (int j0 = n_cand; j0 < nkb; j0 += 64) {
        const int jb = j0 + lane;
        bool take = false;
        if (jb < nkb) {
            const int v = kv_len ? kv_len[jb] : block;
            take = v > 0;
        }
        const unsigned long long bt = __ballot(take);
        if (take) col_idx[base + __popcll(bt & lt_mask)] = jb;
        base += __popcll(bt);
    }
}

// First level of the selection for rows with more than kSegCandidates
// candidates: one wave per (row, segment of kSegCandidates candidates)
// keeps the segment's top min(K_eff, visible) under the same total order
// (key descending, index ascending) and writes them, ascending by index, as
// (order key, candidate index) pairs at slot (row, segment) of the
// workspace, with their count.  A row's top K_eff is among the union of its
// segments' top K_eff.
__global__ void __launch_bounds__(kThreads)
topk_segment_kernel(const double* __restrict__ keys, int rows, int n_cand, int n_seg, int block,
                    const int32_t* __restrict__ kv_len, const int32_t* __restrict__ keff, int seg_cap,
                    unsigned long long* __restrict__ seg_key, int32_t* __restrict__ seg_idx,
                    int32_t* __restrict__ seg_cnt) {
    constexpr int KPL = kSegCandidates / 64;
    __shared__ int hist_all[kThreads / 64][256];
    __shared__ unsigned long long cand_key[kThreads / 64][kSelScratch];
    const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int u = blockIdx.x * (kThreads / 64) + w;
    if (u >= rows * n_seg) return;
    const int r = u / n_seg, sg = u % n_seg;
    const int j0 = sg * kSegCandidates;
    const unsigned long long lt_mask = (1ull << lane) - 1ull;
    const double* row = keys + (int64_t)r * n_cand;
    unsigned long long key[KPL];
    int n_vis = 0;
#pragma unroll
    for (int m = 0; m < KPL; ++m) {
        const int j = j0 + lane + 64 * m;
        double x = 0.0;
        int v = 0;
        if (j < n_cand) {
            x = row[j];
            v = kv_len ? kv_len[j] : block;
        }
        key[m] = v > 0 ? order_key(x) : 0ull;
        n_vis += __popcll(__ballot(key[m] != 0));
    }
    int ke = keff[r];
    ke = ke < n_vis ? ke : n_vis;
    ke = ke < seg_cap ? ke : seg_cap;
    if (lane == 0) seg_cnt[u] = ke;
    if (ke <= 0) return;
    unsigned long long prefix;
    int need;
    bool all_eq;
    select_threshold<KPL>(key, ke, lane, hist_all[w], cand_key[w], prefix, need, all_eq);
    const int64_t base0 = (int64_t)u * seg_cap;
    int base = 0, eq_seen = 0;
#pragma unroll
    for (int m = 0; m < KPL; ++m) {
        const bool gt = key[m] > prefix;
        const bool eq = key[m] != 0 && key[m] == prefix;
        const unsigned long long beq = __ballot(eq);
        const int rank = eq_seen + __popcll(beq & lt_mask);
        eq_seen += __popcll(beq);
        const bool sel = gt || (eq && (all_eq || rank < need));
        const unsigned long long bs = __ballot(sel);
        if (sel) {
            const int64_t at = base0 + base + __popcll(bs & lt_mask);
            seg_key[at] = key[m];
            seg_idx[at] = j0 + lane + 64 * m;
        }
        base += __popcll(bs);
    }
}

// Second level: one wave per row selects its top K_eff among its segments'
// pairs (entry p = segment * seg_cap + e, e < the segment's count; lane l
// holds entries l + 64 m, i.e. ascending candidate index) and writes their
// indices, ascending, after row_ptr[r], then the dense tail.
template <int KPL>
__global__ void __launch_bounds__(kThreads, 3)
topk_merge_kernel(const unsigned long long* __restrict__ seg_key, const int32_t* __restrict__ seg_idx,
                  const int32_t* __restrict__ seg_cnt, int rows, int nqb, int nkb, int n_cand, int n_seg,
                  int seg_cap, int block, const int32_t* __restrict__ q_len, const int32_t* __restrict__ kv_len,
                  const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ keff,
                  int32_t* __restrict__ col_idx) {
    __shared__ int hist_all[kThreads / 64][256];
    __shared__ unsigned long long cand_key[kThreads / 64][kSelScratch];
    const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r = blockIdx.x * (kThreads / 64) + w;
    if (r >= rows) return;
    const int i = r % nqb;
    const int vq = q_len ? q_len[i] : block;
    if (vq <= 0) return;
    const unsigned long long lt_mask = (1ull << lane) - 1ull;
    const int M = n_seg * seg_cap;
    const int64_t base0 = (int64_t)r * M;
    unsigned long long key[KPL];
#pragma unroll
    for (int m = 0; m < KPL; ++m) {
        const int p = lane + 64 * m;
        unsigned long long k = 0ull;
        if (p < M) {
            const int sg = p / seg_cap, e = p - sg * seg_cap;
            if (e < seg_cnt[(int64_t)r * n_seg + sg]) k = seg_key[base0 + p];
        }
        key[m] = k;
    }
    const int ke = keff[r];
    int base = row_ptr[r];
    if (ke > 0) {
        unsigned long long prefix;
        int need;
        bool all_eq;
        select_threshold<KPL>(key, ke, lane, hist_all[w], cand_key[w], prefix, need, all_eq);
        int eq_seen = 0;
#pragma unroll
        for (int m = 0; m < KPL; ++m) {
            const bool gt = key[m] > prefix;
            const bool eq = key[m] != 0 && key[m] == prefix;
            const unsigned long long beq = __ballot(eq);
            const int rank = eq_seen + __popcll(beq & lt_mask);
            eq_seen += __popcll(beq);
            const bool sel = gt || (eq && (all_eq || rank < need));
            const unsigned long long bs = __ballot(sel);
            if (sel) col_idx[base + __popcll(bs & lt_mask)] = seg_idx[base0 + lane + 64 * m];
            base += __popcll(bs);
        }
    }
    for (int j0 = n_cand; j0 < nkb; j0 += 64) {
        const int jb = j0 + lane;
        bool take = false;
        if (jb < nkb) {
            const int v = kv_len ? kv_len[jb] : block;
            take = v > 0;
        }
        const unsigned long long bt = __ballot(take);
        if (take) col_idx[base + __popcll(bt & lt_mask)] = jb;
        base += __popcll(bt);
    }
}

// ------------------------------------------------------------------------
// Route materialisation.
// [Velox: Spatial Memory Makes World Models Efficient -- Methodology,
//  Step 3: a coverage score per query block; Step 4: the geometric fusion
//  applies to well-covered blocks; Step 5: a well-covered query block takes
//  all of the previous chunk's KV blocks, then fills its budget K_cov with
//  the best of the others; a poorly covered one ranks by the unbiased model
//  scores and stops at the shortest prefix whose probability mass passes a
//  threshold, never more than K_unc blocks; either route then adds, outside
//  its budget, the local window and optional reference-frame blocks]
//
// One wave per (head, query block) row builds the row's membership bitmap
// in LDS (one bit per KV block) and writes it out with its population
// count; an exclusive scan turns the counts into row pointers, and a last
// pass writes the set bits of each row, ascending, into its CSR list.

// Largest K_unc: the ordered top-K_unc of a row is ranked in one wave (at
// most four entries per lane).
constexpr int kMaxUnc = kMaxUncovered;

__device__ __forceinline__ double key_value(unsigned long long key) {
    const unsigned long long b = (key & 0x8000000000000000ull) ? (key & 0x7fffffffffffffffull) : ~key;
    return __longlong_as_double((long long)b);
}

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
    for (int m = 32; m > 0; m >>= 1) v += __shfl_xor(v, m);
    return v;
}

template <int KPL>
__global__ void __launch_bounds__(kThreads)
materialize_kernel(const double* __restrict__ keys, int rows, int nqb, int nkb, int block,
                   const int32_t* __restrict__ q_len, const int32_t* __restrict__ kv_len,
                   const float* __restrict__ coverage, double eta_cov, int k_cov, int k_unc, double mass,
                   int prev_begin, int prev_end, const int32_t* __restrict__ window,
                   const int32_t* __restrict__ window_len, int window_stride, int ref_begin, int ref_end,
                   int nwords, uint32_t* __restrict__ bitmap, int32_t* __restrict__ counts) {
    __shared__ int hist_all[kThreads / 64][256];
    __shared__ unsigned long long skey_all[kThreads / 64][kMaxUnc];
    __shared__ int sidx_all[kThreads / 64][kMaxUnc];
    __shared__ uint32_t bits_all[kThreads / 64][kMaxMaterializeBlocks / 32];
    __shared__ unsigned long long cand_all[kThreads / 64][kSelScratch];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int r = blockIdx.x * (kThreads / 64) + w;
    if (r >= rows) return;
    const int i = r % nqb;
    uint32_t* bits = bits_all[w];
    unsigned long long* skey = skey_all[w];
    int* sidx = sidx_all[w];
    const unsigned long long lt_mask = (1ull << lane) - 1ull;
    for (int x = lane; x < nwords; x += 64) bits[x] = 0u;
    __builtin_amdgcn_wave_barrier();
    __asm__ volatile("" ::: "memory");
    const int vq = q_len ? q_len[i] : block;
    if (vq > 0) {
        const bool covered = !coverage || coverage[i] >= (float)eta_cov;
        const double* row = keys + (int64_t)r * nkb;
        // keys of the visible blocks (0: not a candidate); a well-covered row
        // sets the bits of the visible reserved blocks instead
        unsigned long long key[KPL];
        int n_res = 0, n_key = 0;
#pragma unroll
        for (int m = 0; m < KPL; ++m) {
            const int j = lane + 64 * m;
            key[m] = 0;
            bool res = false;
            if (j < nkb && (kv_len ? kv_len[j] : block) > 0) {
                res = covered && j >= prev_begin && j < prev_end;
                if (res)
                    atomicOr(&bits[j >> 5], 1u << (j & 31));
                else
                    key[m] = order_key(row[j]);
            }
            n_res += __popcll(__ballot(res));
            n_key += __popcll(__ballot(key[m] != 0));
        }
        int ke;
        if (covered) {
            const int n_fill = k_cov - n_res > 0 ? k_cov - n_res : 0;
            ke = n_fill < n_key ? n_fill : n_key;
        } else {
            ke = k_unc < n_key ? k_unc : n_key;
        }
        if (ke > 0) {
            unsigned long long prefix;
            int need;
            bool all_eq;
            select_threshold<KPL>(key, ke, lane, hist_all[w], cand_all[w], prefix, need, all_eq);
            __builtin_amdgcn_wave_barrier();
            __asm__ volatile("" ::: "memory");
            // the selected keys in ascending block order: a well-covered row
            // sets their bits, a poorly covered one gathers them for sorting
            int base = 0, eq_seen = 0;
#pragma unroll
            for (int m = 0; m < KPL; ++m) {
                const bool gt = key[m] > prefix;
                const bool eq = key[m] != 0 && key[m] == prefix;
                const unsigned long long beq = __ballot(eq);
                const int rank = eq_seen + __popcll(beq & lt_mask);
                eq_seen += __popcll(beq);
                const bool sel = gt || (eq && rank < need);
                const unsigned long long bs = __ballot(sel);
                if (sel) {
                    const int j = lane + 64 * m;
                    if (covered) {
                        atomicOr(&bits[j >> 5], 1u << (j & 31));
                    } else {
                        const int at = base + __popcll(bs & lt_mask);
                        skey[at] = key[m];
                        sidx[at] = j;
                    }
                }
                base += __popcll(bs);
            }
            if (!covered) {
                // the model distribution p = softmax(s) over the visible
                // blocks: its maximum and normaliser
                unsigned long long kmax = 0;
#pragma unroll
                for (int m = 0; m < KPL; ++m) kmax = key[m] > kmax ? key[m] : kmax;
#pragma unroll
                for (int o = 32; o > 0; o >>= 1) {
                    const unsigned long long ko = shfl_xor_u64(kmax, o);
                    kmax = ko > kmax ? ko : kmax;
                }
                const double smax = key_value(kmax);
                double z = 0.0;
#pragma unroll
                for (int m = 0; m < KPL; ++m)
                    if (key[m] != 0) z += exp(key_value(key[m]) - smax);
                z = wave_sum_f64(z);
                // order the gathered ke keys by rank: an entry's rank is the
                // number of entries before it in selection order (every lane
                // compares its up to four entries with all ke of them)
                __builtin_amdgcn_wave_barrier();
                __asm__ volatile("" ::: "memory");
                constexpr int kPer = kMaxUnc / 64;
                unsigned long long mk[kPer];
                int mi[kPer], rank[kPer];
#pragma unroll
                for (int u = 0; u < kPer; ++u) {
                    const int e = lane + 64 * u;
                    mk[u] = e < ke ? skey[e] : 0ull;
                    mi[u] = e < ke ? sidx[e] : 0x7fffffff;
                    rank[u] = 0;
                }
#pragma unroll 4
                for (int f = 0; f < ke; ++f) {
                    const unsigned long long kf = skey[f];
                    const int jf = sidx[f];
#pragma unroll
                    for (int u = 0; u < kPer; ++u) rank[u] += sel_before(kf, jf, mk[u], mi[u]) ? 1 : 0;
                }
                __builtin_amdgcn_wave_barrier();
                __asm__ volatile("" ::: "memory");
                // p of each entry, in registers at its rank's lane: lane l,
                // slot u holds p of the entry of rank l + 64 u
#pragma unroll
                for (int u = 0; u < kPer; ++u)
                    if (lane + 64 * u < ke) {
                        skey[rank[u]] = mk[u];
                        sidx[rank[u]] = mi[u];
                    }
                __builtin_amdgcn_wave_barrier();
                __asm__ volatile("" ::: "memory");
                double pr[kPer];
#pragma unroll
                for (int u = 0; u < kPer; ++u) {
                    const int e = lane + 64 * u;
                    pr[u] = e < ke ? exp(key_value(skey[e]) - smax) / z : 0.0;
                }
                // shortest prefix, in selection order, whose running sum of p
                // reaches the mass (all ke blocks if none does): a sequential
                // float64 sum, each term read from its lane
                int take = ke;
                double csum = 0.0;
#pragma unroll
                for (int u = 0; u < kPer; ++u) {
                    const int n_u = min(64, ke - 64 * u);
                    const int lo = __double2loint(pr[u]), hi = __double2hiint(pr[u]);
                    for (int l = 0; l < n_u && take == ke; ++l) {
                        csum += __hiloint2double(__builtin_amdgcn_readlane(hi, l), __builtin_amdgcn_readlane(lo, l));
                        if (csum >= mass) take = 64 * u + l + 1;
                    }
                }
                for (int e = lane; e < take; e += 64) atomicOr(&bits[sidx[e] >> 5], 1u << (sidx[e] & 31));
            }
        }
        // the local window and the reference blocks, visible ones only
        if (window) {
            int len = window_len[i];
            len = len < 0 ? 0 : (len > window_stride ? window_stride : len);
            const int32_t* wrow = window + (int64_t)i * window_stride;
            for (int x = lane; x < len; x += 64) {
                const int j = wrow[x];
                if (j >= 0 && j < nkb && (kv_len ? kv_len[j] : block) > 0) atomicOr(&bits[j >> 5], 1u << (j & 31));
            }
        }
        for (int j = ref_begin + lane; j < ref_end; j += 64)
            if ((kv_len ? kv_len[j] : block) > 0) atomicOr(&bits[j >> 5], 1u << (j & 31));
    }
    __builtin_amdgcn_wave_barrier();
    __asm__ volatile("" ::: "memory");
    int cnt = 0;
    for (int x = lane; x < nwords; x += 64) {
        const uint32_t b = bits[x];
        bitmap[(int64_t)r * nwords + x] = b;
        cnt += __popc(b);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) cnt += __shfl_xor(cnt, o);
    if (lane == 0) counts[r] = cnt;
}

// Single workgroup: exclusive prefix sum of the row counts into row_ptr.
__global__ void __launch_bounds__(1024)
scan_counts_kernel(const int32_t* __restrict__ counts, int rows, int32_t* __restrict__ row_ptr) {
    __shared__ int sh[16];
    const int t = threadIdx.x;
    int carry = 0;
    for (int base = 0; base < rows; base += 1024) {
        const int r = base + t;
        const int v = r < rows ? counts[r] : 0;
        int chunk_total;
        const int excl = block_excl_scan_1024(v, sh, &chunk_total);
        if (r < rows) row_ptr[r] = carry + excl;
        carry += chunk_total;
    }
    if (t == 0) row_ptr[rows] = carry;
}

// One wave per row: the set bits of the row's bitmap, ascending, into its
// list.  Lane l owns words l, l + 64, ...; a wave prefix sum of the
// population counts gives each word's write offset.
__global__ void __launch_bounds__(kThreads)
emit_lists_kernel(const uint32_t* __restrict__ bitmap, int rows, int nwords, const int32_t* __restrict__ row_ptr,
                  int32_t* __restrict__ col_idx) {
    const int lane = threadIdx.x & 63;
    const int r = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    if (r >= rows) return;
    int base = row_ptr[r];
    for (int x0 = 0; x0 < nwords; x0 += 64) {
        const int x = x0 + lane;
        uint32_t b = x < nwords ? bitmap[(int64_t)r * nwords + x] : 0u;
        const int c = __popc(b);
        int incl = c;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int up = __shfl_up(incl, off);
            if (lane >= off) incl += up;
        }
        int pos = base + incl - c;
        while (b) {
            const int k = __ffs(b) - 1;
            b &= b - 1;
            col_idx[pos++] = 32 * x + k;
        }
        base += __shfl(incl, 63);
    }
}

}  // namespace

namespace {

// Pooled queries, pooled keys of the candidates not yet cached, the overlap
// row flags (when wanted) and the selection keys of every row; the bias is
// applied only to rows with coverage >= eta_cov when coverage is given.
void launch_pool_score(const bsa_route_args* a, const RouteLayout& lay, void* ws, const float* coverage,
                       double eta_cov, bool want_flags, hipStream_t stream) {
    char* w = static_cast<char*>(ws);
    const double* qbar = a->qpool ? a->qpool : reinterpret_cast<double*>(w + lay.qbar);
    const int64_t qbar_head_stride = a->qpool ? a->qpool_head_stride : (int64_t)a->nqb * a->d;
    const int n_cand = lay.n_cand;
    double* kbar = lay.kbar_in_ws ? reinterpret_cast<double*>(w + lay.kbar) : a->kpool;
    const int64_t kbar_head_blocks = (!lay.kbar_in_ws && a->kpool_head_blocks > 0) ? a->kpool_head_blocks : n_cand;
    double* keys = lay.keys_in_ws ? reinterpret_cast<double*>(w + lay.keys) : a->sel_keys;
    int32_t* flags = reinterpret_cast<int32_t*>(w + lay.flags);
    const bool bf16 = a->dtype == BSA_BF16;

    // pooled queries (unless the caller pooled them)
    if (!a->qpool) {
        double* qout = reinterpret_cast<double*>(w + lay.qbar);
        dim3 grid(a->nqb, a->heads);
        if (bf16)
            hipLaunchKernelGGL(pool_kernel<true>, grid, dim3(kThreads), 0, stream, a->q, a->q_head_stride, a->d,
                               a->block, a->q_block_len, 0, a->nqb, qout, (int64_t)a->nqb);
        else
            hipLaunchKernelGGL(pool_kernel<false>, grid, dim3(kThreads), 0, stream, a->q, a->q_head_stride, a->d,
                               a->block, a->q_block_len, 0, a->nqb, qout, (int64_t)a->nqb);
    }
    // pooled keys of the candidates not yet in the cache
    const int kb0 = a->kpool ? a->kpool_valid_blocks : 0;
    if (n_cand > kb0) {
        const int nb = n_cand - kb0;
        dim3 grid(nb, a->heads);
        if (bf16)
            hipLaunchKernelGGL(pool_kernel<true>, grid, dim3(kThreads), 0, stream, a->k, a->k_head_stride, a->d,
                               a->block, a->kv_block_len, kb0, nb, kbar, kbar_head_blocks);
        else
            hipLaunchKernelGGL(pool_kernel<false>, grid, dim3(kThreads), 0, stream, a->k, a->k_head_stride, a->d,
                               a->block, a->kv_block_len, kb0, nb, kbar, kbar_head_blocks);
    }
    // overlap row flags (for the fallback counts)
    if (want_flags)
        hipLaunchKernelGGL(overlap_flags_kernel, dim3(a->nqb), dim3(kThreads), 0, stream, a->overlap,
                           a->overlap_row_stride, n_cand, a->tau, flags);
    // selection keys
    if (n_cand > 0) {
        dim3 grid((n_cand + kScoreJ - 1) / kScoreJ, a->heads, (a->nqb + kScoreRows - 1) / kScoreRows);
        hipLaunchKernelGGL(score_kernel, grid, dim3(kThreads), 0, stream, qbar, qbar_head_stride, kbar,
                           kbar_head_blocks, a->nqb,
                           n_cand, a->d, a->scale, a->overlap, a->overlap_row_stride, a->lambda, a->g_ref, a->tau,
                           coverage, eta_cov, keys);
    }
}

}  // namespace

hipError_t launch_route(const bsa_route_args* a, const RouteLayout& lay, void* ws, hipStream_t stream) {
    char* w = static_cast<char*>(ws);
    const int n_cand = lay.n_cand;
    double* keys = lay.keys_in_ws ? reinterpret_cast<double*>(w + lay.keys) : a->sel_keys;
    int32_t* keff = reinterpret_cast<int32_t*>(w + lay.keff);
    int32_t* flags = reinterpret_cast<int32_t*>(w + lay.flags);
    const bool want_flags = a->overlap && a->fallback_counts && n_cand > 0;
    // 1-4. pooled queries and keys, overlap flags, selection keys
    launch_pool_score(a, lay, ws, nullptr, 0.0, want_flags, stream);
    // 5. list lengths and row pointers: with one fixed budget (and no
    // overlap rows to count) the selection kernel derives them itself and
    // writes the (zero) fallback counts
    const bool two_level = lay.n_seg > 1;
    const bool fused = !a->k_per_row && !want_flags && a->nqb <= 4096 && !two_level;
    if (!fused)
        hipLaunchKernelGGL(rowptr_kernel, dim3(1), dim3(1024), 0, stream, a->heads, a->nqb, a->nkb, n_cand, a->block,
                           a->q_block_len, a->kv_block_len, a->k_per_row ? 0 : a->k_fixed, a->k_per_row,
                           a->k_max, want_flags ? flags : nullptr, a->row_ptr, keff, a->fallback_counts);
    const int rows = a->heads * a->nqb;
    if (two_level) {
        // 6'. selection in two levels: each segment's top-K, then the top-K
        // over those
        char* wb = static_cast<char*>(ws);
        auto* seg_key = reinterpret_cast<unsigned long long*>(wb + lay.seg_key);
        auto* seg_idx = reinterpret_cast<int32_t*>(wb + lay.seg_idx);
        auto* seg_cnt = reinterpret_cast<int32_t*>(wb + lay.seg_cnt);
        const int units = rows * lay.n_seg;
        hipLaunchKernelGGL(topk_segment_kernel, dim3((units + kThreads / 64 - 1) / (kThreads / 64)), dim3(kThreads),
                           0, stream, keys, rows, n_cand, lay.n_seg, a->block, a->kv_block_len, keff, lay.seg_cap,
                           seg_key, seg_idx, seg_cnt);
        const dim3 mgrid((rows + kThreads / 64 - 1) / (kThreads / 64));
        const int M = lay.n_seg * lay.seg_cap;
#define BSA_MERGE(KPL)                                                                                          \
    hipLaunchKernelGGL(topk_merge_kernel<KPL>, mgrid, dim3(kThreads), 0, stream, seg_key, seg_idx, seg_cnt, rows, \
                       a->nqb, a->nkb, n_cand, lay.n_seg, lay.seg_cap, a->block, a->q_block_len, a->kv_block_len, \
                       a->row_ptr, keff, a->col_idx)
        if (M <= 64 * 8)
            BSA_MERGE(8);
        else if (M <= 64 * 16)
            BSA_MERGE(16);
        else if (M <= 64 * 32)
            BSA_MERGE(32);
        else
            BSA_MERGE(64);
#undef BSA_MERGE
        return hipGetLastError();
    }
    // 6. selection: one wave per row
    const int k_fused = fused ? a->k_fixed : -1;
    const dim3 grid((rows + kThreads / 64 - 1) / (kThreads / 64));
#define BSA_TOPK(KPL)                                                                                       \
    hipLaunchKernelGGL(topk_kernel<KPL>, grid, dim3(kThreads), 0, stream, keys, rows, a->nqb, n_cand, a->nkb, \
                       a->block, a->q_block_len, a->kv_block_len, k_fused, a->row_ptr, keff, a->col_idx,    \
                       fused ? a->fallback_counts : nullptr)
    if (n_cand <= 64 * 8)
        BSA_TOPK(8);
    else if (n_cand <= 64 * 16)
        BSA_TOPK(16);
    else if (n_cand <= 64 * 24)
        BSA_TOPK(24);
    else if (n_cand <= 64 * 32)
        BSA_TOPK(32);
    else if (n_cand <= 64 * 40)
        BSA_TOPK(40);
    else if (n_cand <= 64 * 48)
        BSA_TOPK(48);
    else
        BSA_TOPK(64);
#undef BSA_TOPK
    return hipGetLastError();
}

hipError_t launch_materialize(const bsa_route_args* a, const bsa_materialize_args* m, const RouteLayout& lay,
                              void* ws, hipStream_t stream) {
    char* w = static_cast<char*>(ws);
    const double* keys = lay.keys_in_ws ? reinterpret_cast<const double*>(w + lay.keys) : a->sel_keys;
    uint32_t* bitmap = reinterpret_cast<uint32_t*>(w + lay.bitmap);
    int32_t* counts = reinterpret_cast<int32_t*>(w + lay.counts);
    const int nkb = a->nkb, rows = a->heads * a->nqb;
    const int nwords = (nkb + 31) / 32;
    launch_pool_score(a, lay, ws, m->coverage, m->eta_cov, false, stream);
    const int pb = m->prev_begin < nkb ? m->prev_begin : nkb, pe = m->prev_end < nkb ? m->prev_end : nkb;
    const int rb = m->ref_begin < nkb ? m->ref_begin : nkb, re = m->ref_end < nkb ? m->ref_end : nkb;
    const dim3 grid((rows + kThreads / 64 - 1) / (kThreads / 64));
#define BSA_MAT(KPL)                                                                                            \
    hipLaunchKernelGGL(materialize_kernel<KPL>, grid, dim3(kThreads), 0, stream, keys, rows, a->nqb, nkb,        \
                       a->block, a->q_block_len, a->kv_block_len, m->coverage, m->eta_cov, m->k_cov, m->k_unc,  \
                       m->mass, pb, pe, m->window, m->window_len, m->window_stride, rb, re, nwords, bitmap, counts)
    // no 16-key-per-lane instance: the register allocator spills that one
    // to scratch, so rows of 513..1536 blocks take the 24-key instance
    if (nkb <= 64 * 8)
        BSA_MAT(8);
    else if (nkb <= 64 * 24)
        BSA_MAT(24);
    else if (nkb <= 64 * 32)
        BSA_MAT(32);
    else if (nkb <= 64 * 40)
        BSA_MAT(40);
    else if (nkb <= 64 * 48)
        BSA_MAT(48);
    else
        BSA_MAT(64);
#undef BSA_MAT
    hipLaunchKernelGGL(scan_counts_kernel, dim3(1), dim3(1024), 0, stream, counts, rows, a->row_ptr);
    hipLaunchKernelGGL(emit_lists_kernel, grid, dim3(kThreads), 0, stream, bitmap, rows, nwords, a->row_ptr,
                       a->col_idx);
    return hipGetLastError();
}

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device (null until looked up)

}  // namespace

hipError_t static_route_scratch(void** ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace bsa
