// Indexed block-sparse attention (and the dense case through the same code).
//
// [Velox: Spatial Memory Makes World Models Efficient -- Methodology, Step 6:
//  an indexed block-sparse attention kernel, not a dense call with a mask;
//  the block is the attention tile, so a skipped block costs neither its
//  QK^T tile product nor its KV tile load; Main Findings: dense attention
//  over all retained context is the baseline]
// [Light Interaction -- abstract: 3-D block-sparse attention]
//
// One workgroup owns one (head, query block).  It walks the block's list of
// KV blocks; for each it stages the K tile (row-major) and the V tile
// (transposed, keys contiguous) in LDS and every wave multiplies them with
// its 32 query rows on the matrix cores:
//
//   S^T = K Q^T   v_mfma_f32_32x32x16_bf16, A = K rows from LDS, B = Q^T
//                 fragments held in registers for the whole walk.  The
//                 32x32 result puts one query per lane column, so each lane
//                 holds half of its query's scores and the row maximum /
//                 sum need only one cross-lane exchange (lane ^ 32).
//   O^T += V^T P^T  A = V^T rows from LDS, B = P^T straight from the S^T
//                 registers (rounded to bf16).  The order of keys inside a
//                 32-key tile is permuted when K rows are read so that each
//                 lane's 8 probabilities for one k-step are 8 consecutive
//                 keys, i.e. one 16-byte read of V^T.
//
// The softmax is online (running max m and sum l per query, base-2
// exponentials with the scale folded in), in fp32.  Padded keys are masked
// to -inf, padded query rows are written as zeros, an empty list gives zeros
// and LSE = -inf.  Waves whose 32 query rows are all padding skip the math.
// The output rows can also go straight to raster token order through a row
// map (the inverse of the forward permutation, fused into the epilogue).
#include <hip/hip_runtime.h>

#include <type_traits>

#include "kernels.h"

namespace bsa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

struct AttnArgs {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    int heads, nqb, nkb;
    int64_t q_hs, k_hs, v_hs, o_hs;
    const int32_t* q_len;
    const int32_t* kv_len;
    const int32_t* row_ptr;
    const int32_t* col_idx;
    int64_t col_len;
    float scale;       // natural-log scale of the scores
    float scale_log2;  // scale * log2(e)
    // raster output (o_map non-NULL): query row g = i*BLK + r of head h goes
    // to o[o_map[g] * o_ts + h * D] when g < o_map_len and o_map[g] >= 0;
    // other rows (padding) are not written
    const int32_t* o_map;
    int o_map_len;
    int64_t o_ts;
    // raster queries (q_map non-NULL): query row g of head h is read from
    // q[q_map[g] * q_ts + h * D]; rows past q_map_len or mapped to a
    // negative entry (padding) read as zeros
    const int32_t* q_map;
    int q_map_len;
    int64_t q_ts;
};

// Query row of (head h, query row g): the head-major blocked row, or the
// raster token row through the map (nullptr: a padding row, read as zeros).
template <typename T>
__device__ __forceinline__ const T* in_row(const AttnArgs& a, int h, int64_t g, int D) {
    if (!a.q_map) return static_cast<const T*>(a.q) + h * a.q_hs + g * D;
    const int t = g < a.q_map_len ? a.q_map[g] : -1;
    return t < 0 ? nullptr : static_cast<const T*>(a.q) + (int64_t)t * a.q_ts + (int64_t)h * D;
}

// Output row of (head h, query row g): the head-major blocked row, or the
// raster token row through the map (nullptr: a padding row, not written).
template <typename T>
__device__ __forceinline__ T* out_row(const AttnArgs& a, int h, int64_t g, int D) {
    if (!a.o_map) return static_cast<T*>(a.o) + h * a.o_hs + g * D;
    const int t = g < a.o_map_len ? a.o_map[g] : -1;
    return t < 0 ? nullptr : static_cast<T*>(a.o) + (int64_t)t * a.o_ts + (int64_t)h * D;
}

constexpr float kLn2 = 0.69314718055994530942f;

// Workgroup -> (head, query block).  Workgroups are dispatched round-robin
// over the 8 XCDs; remap so that each XCD receives a contiguous run of
// (head, query block) items, keeping a head's KV blocks in one L2.
__device__ __forceinline__ void map_item(int total, int nqb, int& h, int& i) {
    const int b = blockIdx.x;
    const int per = total / 8;
    const int item = b < per * 8 ? (b % 8) * per + b / 8 : b;
    h = item / nqb;
    i = item % nqb;
}

// Workgroup -> item for routed lists: the XCD runs of map_item, but inside
// a run the query blocks of one head (in windows of at most 128) start
// longest list first, ties to the lower index.  The workgroups that share
// an XCD at any time then walk lists of similar length and reach the blocks
// they have in common (notably a dense tail at the end of every list) at
// similar times, while those blocks are still in that XCD's L2; the longest
// lists also no longer start last.  The order is a permutation of the
// window (strict order on (length, index)), found by every wave alone from
// the window's row pointers: rank = number of items ahead of it.
__device__ __forceinline__ int longest_first_item(const int32_t* row_ptr, int64_t col_len, int total, int nqb) {
    constexpr int kWin = 128;
    const int b = blockIdx.x;
    const int per = total / 8;
    if (b >= per * 8) return b;
    const int run = (b % 8) * per, item0 = run + b / 8;
    const int hs = item0 / nqb * nqb;
    const int lo = run > hs ? run : hs;
    const int hi = run + per < hs + nqb ? run + per : hs + nqb;
    const int ws = lo + (item0 - lo) / kWin * kWin;
    const int n = hi - ws < kWin ? hi - ws : kWin;
    const int r = item0 - ws;
    const int lane = threadIdx.x & 63;
    // key: length (clamped to 2^24 - 1) above the inverted window index, so
    // a larger key goes first and keys are distinct
    uint32_t key[2];
#pragma unroll
    for (int w = 0; w < 2; ++w) {
        const int t = lane + 64 * w;
        uint32_t len = 0;
        if (t < n) {
            int e0 = row_ptr[ws + t], e1 = row_ptr[ws + t + 1];
            e0 = e0 < 0 ? 0 : e0;
            e1 = e1 > col_len ? (int)col_len : e1;
            len = e1 > e0 ? (uint32_t)(e1 - e0) : 0u;
            len = len < (1u << 24) ? len : (1u << 24) - 1u;
        }
        key[w] = (len << 7) | (uint32_t)(kWin - 1 - t);
    }
    int rank[2] = {0, 0};
    for (int k = 0; k < n; ++k) {
        const uint32_t kk = k < 64 ? (uint32_t)__builtin_amdgcn_readlane((int)key[0], k)
                                   : (uint32_t)__builtin_amdgcn_readlane((int)key[1], k - 64);
        rank[0] += kk > key[0];
        rank[1] += kk > key[1];
    }
#pragma unroll
    for (int w = 0; w < 2; ++w) {
        const uint64_t m = __ballot(lane + 64 * w < n && rank[w] == r);
        if (m) return __builtin_amdgcn_readfirstlane(ws + 64 * w + __builtin_ctzll(m));
    }
    return item0;  // unreachable: the ranks are a permutation of [0, n)
}

__device__ __forceinline__ bf16x8_t lds_bf16x8(const uint16_t* p) {
    return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(p));
}

// Row of a 32-key tile that MFMA row m reads (see the header comment).
__device__ __forceinline__ int key_of_row(int m) {
    const int g = m >> 3, hh = (m >> 2) & 1, ii = m & 3;
    return 16 * (g >> 1) + 8 * hh + 4 * (g & 1) + ii;
}

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
typedef __attribute__((address_space(3))) uint16_t lds_u16_t;
typedef const __attribute__((address_space(4))) int32_t const_i32_t;

constexpr int kSubKeys = 32;  // keys per pipeline stage (sub-tile)
constexpr float kRescaleSlack = 8.0f;  // log2 units the running max may lag

// LDS sub-tile layout: kSubKeys rows of D bf16 (no padding), 16-byte chunks
// XOR-swizzled by row.  K tiles are read by ds_read_b128 with 16 lanes per
// LDS cycle touching 16 different rows at one chunk: XOR with row % 16
// spreads them over all bank groups.  V tiles are read by transposing 8-byte
// reads in which 32 lanes touch 4 consecutive rows x 4 consecutive chunks:
// XOR with 4 * (row % 4) (d = 128; 4 * (row/2 % 2) for d = 64, two rows per
// bank period) gives those 16 chunk accesses 16 distinct bank groups.
template <int D, bool IS_V>
__device__ __forceinline__ int swz(int row) {
    constexpr int CPR = D / 8;  // chunks per row
    if (!IS_V) return row & (CPR - 1);
    return D == 128 ? 4 * (row & 3) : 4 * ((row >> 1) & 1);
}

template <int D, bool IS_V>
__device__ __forceinline__ int tile_off(int row, int c) {
    return row * (D * 2) + ((c ^ swz<D, IS_V>(row)) << 4);
}

// Per-lane byte offsets of the direct global -> LDS copy of one
// kSubKeys x D bf16 sub-tile into the swizzled layout.  One 16-byte buffer
// load per lane lands at the LDS address in M0 + 16 * lane, so lane l of
// wave-instruction I fills row I * RPI + l / CPR, physical chunk l % CPR, and
// fetches the logical chunk that belongs there.  The offsets do not depend
// on the block, so they are computed once.
template <int D, int NW, bool IS_V>
__device__ __forceinline__ uint32_t dma_lane_offset(int n, int wave, int lane) {
    constexpr int CPR = D / 8;
    constexpr int RPI = 64 / CPR;  // rows per wave-instruction (1 KB)
    const int I = n * NW + wave;
    const int row = I * RPI + lane / CPR;
    const int c = (lane % CPR) ^ swz<D, IS_V>(row);
    return (uint32_t)(row * D + c * 8) * 2u;
}

// Instruction n's lane offset equals instruction 0's plus n * NW KB when
// the NW * RPI rows that one instruction round covers are a whole number of
// swizzle periods (16 rows for K, 4 for V at d = 128).
template <int D, int NW>
constexpr bool dma_lane_offset_step() {
    return D == 128 && (NW * (64 / (D / 8))) % 16 == 0;
}

// Issue the copies of one sub-tile: NI wave-instructions; buffer resource =
// the block, bounded to its valid rows; scalar offset = the sub-tile, vector
// offset = the lane's.  The bound applies to the whole offset (scalar +
// vector): rows past it are not fetched and land in LDS as zeros.
template <int NI, int NW, bool FORM_AT_USE = false>
__device__ __forceinline__ void dma_issue(__amdgpu_buffer_rsrc_t rsrc, uint32_t sub_off, const uint32_t* voff,
                                          uint16_t* lds_tile, int wave) {
    if constexpr (FORM_AT_USE) {
        // For a kernel short of registers: the LDS destination is formed
        // here from one wave-uniform base that passes through an empty asm
        // (otherwise the compiler keeps every (buffer, instruction) address
        // of the unrolled loop live in scalar registers), and instruction n
        // reuses the lane offset of instruction 0 with n * NW * 1 KB more in
        // the scalar offset (see dma_lane_offset_step).
        constexpr uint32_t kStep = (uint32_t)NW * 1024u;
        uint32_t base = (uint32_t)(uintptr_t)(lds_u16_t*)lds_tile + (uint32_t)wave * 1024u;
        __asm__ volatile("" : "+s"(base));
#pragma unroll
        for (int n = 0; n < NI; ++n)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rsrc, (__attribute__((address_space(3))) void*)(uintptr_t)(base + n * kStep), 16, voff[0],
                sub_off + n * kStep, 0, 0);
    } else {
#pragma unroll
        for (int n = 0; n < NI; ++n)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rsrc, (__attribute__((address_space(3))) void*)((lds_u16_t*)lds_tile + (n * NW + wave) * 512), 16,
                voff[n], sub_off, 0, 0);
    }
}

// Raw buffer (no stride) over nbytes from base; 0x00020000 = 32-bit data
// format (untyped loads).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t block_rsrc(const uint16_t* base, uint32_t nbytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base), 0, (int)nbytes, 0x00020000);
}

// Plain v_max3_f32 / v_max_f32.  fmaxf must quiet signalling NaNs, so the
// compiler canonicalises both inputs first (two extra instructions per
// maximum); the scores here are MFMA and FMA results (never signalling), so
// the bare instructions give the same maxima.
__device__ __forceinline__ float max3_raw(float a, float b, float c) {
    float r;
    __asm__("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

// max over the two lanes l and l ^ 32 (which hold one query's two key halves)
__device__ __forceinline__ float max_halves(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    float m;
    __asm__("v_max_f32 %0, %1, %2" : "=v"(m) : "v"(__uint_as_float(r[0])), "v"(__uint_as_float(r[1])));
    return m;
}

__device__ __forceinline__ float add_halves(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Workgroup barrier for the copy pipeline.  A fenced barrier
// (__syncthreads, or an LDS-scoped fence, since LDS-DMA writes are pending
// LDS writes) makes the compiler drain every outstanding copy, including the
// stages still streaming in.  Here each wave has already waited (vmcnt) for
// its own copies of the stages about to be read, and every read of the stages
// about to be overwritten was consumed by an MFMA before the barrier, so a
// bare s_barrier is enough; the empty asm statements only stop the compiler
// from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
}

// s_waitcnt lgkmcnt(0) alone (vmcnt and expcnt fields at their maxima)
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4)); }

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    // gfx9 s_waitcnt: vmcnt[3:0] and [15:14], expcnt[6:4] (7 = no wait),
    // lgkmcnt[11:8] (15 = no wait)
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Reader of one row's list of KV blocks.  next() returns the next in-range
// block and its valid-key count (clamped to [0, BLK]), or -1 at the end.
// The scalar loads for the following entry are issued by prefetch1() (its
// block index) and prefetch2() (its key count, which needs the index) at the
// end of the two iterations after a next(), and waited for at the top of the
// next iteration, where no LDS read is in flight: a scalar load pending
// during the LDS reads would force every LDS wait to lgkmcnt(0), since
// scalar loads complete out of order.  Out-of-range entries take a slow
// path with direct loads.
//
// With PIPE2 (a new block every iteration) the block index is loaded one
// entry further ahead (pj2), so that the two loads issued after a next()
// by prefetch_both() -- the key count of the next entry and the index of
// the one after -- do not depend on each other.
template <int BLK, bool DENSE, bool PIPE2 = false>
struct ListReader {
    const_i32_t* col;
    const_i32_t* kvl;
    int e, e1, nkb, pj, pv, pj2 = 0;
    __device__ __forceinline__ int keys(int v) const {
        return __builtin_amdgcn_readfirstlane(v < 0 ? 0 : (v > BLK ? BLK : v));
    }
    __device__ __forceinline__ int clamp_j(int j) const { return j < 0 ? 0 : (j >= nkb ? nkb - 1 : j); }
    __device__ __forceinline__ void init(const_i32_t* c, const_i32_t* kv, int e0_, int e1_, int nkb_) {
        col = c;
        kvl = kv;
        e = e0_;
        e1 = e1_;
        nkb = nkb_;
        pj = DENSE ? e : (e < e1 ? col[e] : 0);
        pv = kvl ? kvl[clamp_j(pj)] : BLK;
        if (PIPE2) pj2 = DENSE ? e + 1 : (e + 1 < e1 ? col[e + 1] : 0);
    }
    // PIPE2: after a next(), the entry now at e and the index of e + 1
    __device__ __forceinline__ void prefetch_both() {
        pv = kvl ? kvl[clamp_j(pj2)] : BLK;
        pj = pj2;
        pj2 = DENSE ? e + 1 : col[e + 1 < e1 ? e + 1 : e1 - 1];
    }
    __device__ __forceinline__ void prefetch1() {
        pj = DENSE ? e : col[e < e1 ? e : e1 - 1];
    }
    __device__ __forceinline__ void prefetch2() {
        if (kvl) pv = kvl[clamp_j(pj)];
    }
    __device__ __forceinline__ int next(int& vk) {
        if (e >= e1) return -1;
        int j = pj;
        vk = keys(pv);
        ++e;
        if (__builtin_expect(j < 0 || j >= nkb, 0)) {
            j = -1;
            while (e < e1) {
                const int jj = col[e++];
                if (jj >= 0 && jj < nkb) {
                    j = jj;
                    vk = keys(kvl ? kvl[jj] : BLK);
                    break;
                }
            }
            if (PIPE2) pj2 = col[e < e1 ? e : e1 - 1];  // the entry at e, for prefetch_both
        }
        return j;
    }
};

// Compile-time loop: f(integral_constant<int, I>) for I in [B, E).
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>());
        static_for<B + 1, E>(f);
    }
}

// Waves that share each 32-row query tile, each taking its own 32 keys of
// every slot: 2 for the 64-row, d-128 workgroup (four waves instead of two,
// so two workgroups per CU give each SIMD two waves), 1 otherwise.
constexpr int attn_key_split(int blk, int d) { return blk == 64 && d == 128 ? 2 : 1; }

// Compile-time loop that stops at the first f(integral_constant<int, I>)
// returning false; true when every call did.
template <int B, int E, class F>
__device__ __forceinline__ bool static_all(F&& f) {
    if constexpr (B < E) {
        if (!f(std::integral_constant<int, B>())) return false;
        return static_all<B + 1, E>(f);
    }
    return true;
}

constexpr int gcd_c(int x, int y) { return y == 0 ? x : gcd_c(y, x % y); }
constexpr int lcm3(int x, int y, int z) {
    const int xy = x / gcd_c(x, y) * y;
    return xy / gcd_c(xy, z) * z;
}

// Scheduling fence: the compiler keeps the instruction order across it.
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// Workgroup of BLK/32 query tiles of 32 rows, one (head, query block).
// Keys stream in slots of SLOTK keys: slot t is slot t % SUBS of the
// t / SUBS-th listed block.  K and V have rings of RK and RV slots, sized so
// that every SIMD holds two waves, whose softmax and matrix work then
// overlap each other:
//  - 128 rows: four waves, one per query tile, 32-key slots, rings of four
//    K and four V slots (2 x 32 KB at d = 128, two workgroups per CU);
//  - 64 rows at d = 128: four waves, two per query tile, each taking its
//    own 32 keys of every 64-key slot (one slot = one block), rings of two
//    K and two V slots (64 KB, two workgroups per CU).  The two waves of a
//    tile keep separate softmax states, merged at the end.  A two-wave
//    workgroup with the same 64 KB would leave one wave per SIMD; with a
//    smaller ring (four per CU) twice the workgroups share each XCD's L2;
//  - d = 64: 32-key slots, four of each (32 KB).
//
// Iteration t, after one barrier:
//   copies      V of slot t+RV-1, then K of slot t+RK, are issued into the
//               buffers freed by iteration t-1;
//   phase A     S(t+1) = K(t+1) Q^T on the matrix cores while the vector
//               units exponentiate slot t's scores into bf16 P(t);
//   phase B     O^T += V(t)^T P(t)^T on the matrix cores while the vector
//               units scale S(t+1) into base-2 logits, take its row maximum
//               and add P(t) into the running row sums.
// The running reference max per query moves only when a sub-tile's maximum
// passes it by more than kRescaleSlack (a rare, wave-uniform branch), so
// p <= 2^slack and each query's arithmetic depends on its own scores only.
template <int BLK, int D, bool DENSE>
__global__ void __launch_bounds__(BLK * 2 * attn_key_split(BLK, D), 2) attn_bf16_kernel(AttnArgs a) {
    constexpr int KS = attn_key_split(BLK, D);  // waves per query tile, one key share each
    constexpr int NWQ = BLK / 32;               // query tiles (32 rows each)
    constexpr int NW = NWQ * KS;                // waves
    constexpr int DT = D / 32, KK = D / 16;
    constexpr int SLOTK = kSubKeys * KS;        // keys per slot (one pipeline stage)
    constexpr int SUBE = SLOTK * D;             // elements of a K or V slot buffer
    constexpr int SUBS = BLK / SLOTK;           // slots per block
    constexpr int NI = SLOTK * D * 2 / 1024 / NW;  // copy instructions per wave per slot
    constexpr int RK = KS == 2 ? 2 : 4, RV = KS == 2 ? 2 : 4;  // K and V ring depths (slots)
    constexpr int LAG = (RK - 1) / SUBS;        // blocks between the K-copy cursor and slot t+1
    constexpr int VLAG = (RK - RV) / SUBS;      // blocks between it and a V copy that opens a block
    constexpr int HD = LAG + 1;                 // depth of the cursor history
    constexpr int U = lcm3(RK, RV, SUBS);       // unroll period: every ring index a constant
    static_assert(SLOTK * D * 2 % (1024 * NW) == 0, "slot copy must split evenly over the waves");
    static_assert(RK >= RV && LAG <= 2 && VLAG <= LAG, "cursor history");
    // one LDS object per buffer: the compiler then tracks each buffer's
    // copies on their own (a read of one waits only for that buffer's)
    __shared__ __attribute__((aligned(1024))) uint16_t kb0[SUBE], kb1[SUBE], kb2[SUBE], kb3[RK > 3 ? SUBE : 1];
    __shared__ __attribute__((aligned(1024))) uint16_t vb0[SUBE], vb1[SUBE], vb2[RV > 2 ? SUBE : 1],
        vb3[RV > 3 ? SUBE : 1];
    uint16_t* const KB[4] = {kb0, kb1, kb2, kb3};
    uint16_t* const VB[4] = {vb0, vb1, vb2, vb3};

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ks = KS == 1 ? 0 : wave / NWQ;                    // this wave's key share of a slot
    const int ksoff = ks * kSubKeys * D * 2;                    // bytes to its 32 keys in a slot buffer
    const int hi = lane >> 5, l32 = lane & 31, g16 = lane & 15;
    int h, i;
    if (DENSE) {
        map_item(a.heads * a.nqb, a.nqb, h, i);
    } else {
        const int item = longest_first_item(a.row_ptr, a.col_len, a.heads * a.nqb, a.nqb);
        h = item / a.nqb;
        i = item % a.nqb;
    }
    int vq = a.q_len ? a.q_len[i] : BLK;
    vq = vq < 0 ? 0 : (vq > BLK ? BLK : vq);
    const int q0 = (wave % NWQ) * 32;
    const bool active = q0 < vq;
    const bool valid_row = q0 + l32 < vq;

    const uint16_t* Kh = static_cast<const uint16_t*>(a.k) + h * a.k_hs;
    const uint16_t* Vh = static_cast<const uint16_t*>(a.v) + h * a.v_hs;

    // Q^T fragments (B operand of S^T = K Q^T), held for the whole walk
    bf16x8_t qf[KK];
    {
        const uint16_t* qrow = in_row<uint16_t>(a, h, (int64_t)i * BLK + q0 + l32, D);
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
            qf[kk] = qrow ? lds_bf16x8(qrow + 8 * hi + 16 * kk) : bf16x8_t{};
    }

    int e0, e1;
    if (DENSE) {
        e0 = 0;
        e1 = a.nkb;
    } else {
        const int row = h * a.nqb + i;
        const_i32_t* rp = (const_i32_t*)a.row_ptr;
        e0 = rp[row];
        e1 = rp[row + 1];
        e0 = e0 < 0 ? 0 : e0;
        e1 = e1 > a.col_len ? (int)a.col_len : e1;
    }
    ListReader<BLK, DENSE, SUBS == 1> list;
    list.init((const_i32_t*)a.col_idx, (const_i32_t*)a.kv_len, e0, e1, a.nkb);

    // K-copy cursor: block jk; the blocks it has entered are published to a
    // two-deep history (j, valid keys; -1 keys past the end) that the V-copy
    // cursor (same block) and the compute cursor (LAG blocks behind) read.
    int jk, h0v;
    jk = list.next(h0v);
    if (jk < 0) {
        // empty list: zeros and -inf, no copies in flight
        const int qrow = q0 + l32;
        uint16_t* Orow = out_row<uint16_t>(a, h, (int64_t)i * BLK + qrow, D);
        if (Orow)
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    *reinterpret_cast<uint2*>(Orow + dt * 32 + 8 * g + 4 * hi) = make_uint2(0u, 0u);
        if (a.lse && hi == 0) a.lse[(int64_t)h * a.nqb * BLK + (int64_t)i * BLK + qrow] = -INFINITY;
        return;
    }
    // history: [0] = the K-copy cursor's block, [d] = d blocks before it:
    // its index and valid keys, -1 keys past the end of the list (ints, kept
    // in scalar registers)
    int hj[HD], hv[HD];
    hj[0] = jk, hv[0] = h0v;
#pragma unroll
    for (int d = 1; d < HD; ++d) hj[d] = jk, hv[d] = -1;
    auto k_advance = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int d = HD - 1; d > 0; --d) hj[d] = hj[d - 1], hv[d] = hv[d - 1];
        int nv = 0;
        const int nj = hv[0] < 0 ? -1 : list.next(nv);
        if (nj >= 0) {
            jk = nj;
            hv[0] = nv;
        } else {
            hv[0] = -1;  // copies past the end fetch nothing (never computed)
        }
        hj[0] = jk;
    };
    // the list's next entry: two loads (see ListReader)
    auto prefetch_all = [&]() __attribute__((always_inline)) {
        if constexpr (SUBS == 1) {
            list.prefetch_both();
        } else {
            list.prefetch1();
            list.prefetch2();
        }
    };
    int kvk = 0, vvk = 0;  // valid keys of the blocks being copied (0 past the end)
    int jv = jk;

    static_assert(KS == 1 || dma_lane_offset_step<D, NW>(), "copy offsets of the key-split kernel");
    uint32_t koffs[NI], voffs[NI];
#pragma unroll
    for (int n = 0; n < NI; ++n) {
        koffs[n] = dma_lane_offset<D, NW, false>(n, wave, lane);
        voffs[n] = dma_lane_offset<D, NW, true>(n, wave, lane);
    }
    constexpr uint32_t kSubBytes = SLOTK * D * 2;
    // copies of one slot, bounded to the block's valid rows: padded rows
    // and copies past the end of the list (0 valid keys) fetch nothing
    auto issue_k = [&](int buf, int sub) __attribute__((always_inline)) {
        kvk = hv[0] < 0 ? 0 : hv[0];
        dma_issue<NI, NW, KS == 2>(block_rsrc(Kh + (int64_t)jk * BLK * D, (uint32_t)kvk * (D * 2)), sub * kSubBytes, koffs,
                          KB[buf], wave);
    };
    auto issue_v = [&](int buf, int sub) __attribute__((always_inline)) {
        dma_issue<NI, NW, KS == 2>(block_rsrc(Vh + (int64_t)jv * BLK * D, (uint32_t)vvk * (D * 2)), sub * kSubBytes, voffs,
                          VB[buf], wave);
    };

    // prologue: K of slots 0..RK-1, V of slots 0..RV-2
    prefetch_all();
#pragma unroll
    for (int s = 0; s < RK; ++s) {
        if (s > 0 && s % SUBS == 0) {
            k_advance();
            prefetch_all();
        }
        issue_k(s, s % SUBS);
        if (s < RV - 1) {
            if (s % SUBS == 0) {  // the V copy follows the K copy of its slot
                jv = hj[0];
                vvk = hv[0] < 0 ? 0 : hv[0];
            }
            issue_v(s, s % SUBS);
        }
    }

    // per-lane LDS byte offsets (loop invariant)
    const int kr = key_of_row(l32);
    int koff[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) koff[kk] = tile_off<D, false>(kr, 2 * kk + hi) + ksoff;
    int voff[DT][2];
    {
        const int j4 = g16 >> 2, r4 = g16 & 3, g2 = (lane >> 4) & 1;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int h4 = 0; h4 < 2; ++h4) {
                const int row = 8 * hi + 4 * h4 + j4;  // + 16*s2
                const int col = dt * 32 + 16 * g2 + 4 * r4;
                voff[dt][h4] = tile_off<D, true>(row, col >> 3) + ((col >> 2) & 1) * 8 + ksoff;
            }
    }

    f32x16_t o[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;
    float ref = 0.f, l = 0.f;  // reference max (base-2 logit units) and partial row sum
    bool ref_set = false;
    const float c2 = a.scale_log2;
    f32x16_t xc;  // base-2 logits of slot t relative to ref

    auto scores = [&](const uint16_t* kbuf) __attribute__((always_inline)) {
        const char* base = reinterpret_cast<const char*>(kbuf);
        bf16x8_t kf[KK];
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
            kf[kk] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(base + koff[kk]));
        f32x16_t s;
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kk], qf[kk], s, 0, 0, 0);
        return s;
    };
    // lane holds keys 16*(r/8) + 8*hi + (r%8) of the sub-tile
    auto mask = [&](f32x16_t& s, int nv) __attribute__((always_inline)) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int key = 16 * (r >> 3) + 8 * hi + (r & 7);
            if (key >= nv) s[r] = -INFINITY;
        }
    };
    auto load_v = [&](const uint16_t* vbuf, s16x4_t (&vr)[2][DT][2]) {
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int h4 = 0; h4 < 2; ++h4)
                    vr[s2][dt][h4] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_s16x4_t*)((__attribute__((address_space(3))) char*)vbuf + voff[dt][h4] +
                                       s2 * 16 * D * 2));
    };
    // bf16 P of slot t and its fp32 row sum
    auto exp_p = [&](bf16x8_t (&pf)[2]) __attribute__((always_inline)) {
        float ls = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float p = __builtin_amdgcn_exp2f(xc[r]);
            ls += p;
            pf[r >> 3][r & 7] = (__bf16)p;
        }
        l += ls;
    };
    auto pv = [&](const s16x4_t (&vr)[2][DT][2], const bf16x8_t (&pf)[2]) {
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const bf16x8_t vf = __builtin_bit_cast(
                    bf16x8_t, __builtin_shufflevector(vr[s2][dt][0], vr[s2][dt][1], 0, 1, 2, 3, 4, 5, 6, 7));
                o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[s2], o[dt], 0, 0, 0);
            }
    };
    // scale raw scores into logits relative to ref and take this lane's
    // maximum (half of its query's keys); then move ref (rare, wave-uniform
    // branch) where the sub-tile's maximum passes it by more than the slack,
    // or first sets it.  The common path compares each lane's own maximum
    // with its query's threshold thr_l (+inf for padded rows): a query needs
    // a move exactly when one of its two lanes passes, so the cross-lane
    // maximum is only taken on the rare path.
    float m3l = -INFINITY;
    float thr_l = valid_row ? -INFINITY : INFINITY;
    auto logits_scale = [&](const f32x16_t& s) __attribute__((always_inline)) {
        float m3 = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            xc[r] = fmaf(s[r], c2, -ref);
            m3 = fmaxf(m3, xc[r]);
        }
        m3l = m3;
    };
    auto logits_check = [&]() __attribute__((always_inline)) {
        if (__any(m3l > thr_l)) {
            const float mx = max_halves(m3l);
            const float thr = ref_set ? kRescaleSlack : -INFINITY;
            const bool need = valid_row & (mx > thr);
            const float shift = need ? mx : 0.f;
            const float alpha = (need && ref_set) ? __builtin_amdgcn_exp2f(-shift) : 1.0f;
            ref += shift;
            ref_set = ref_set || need;
            thr_l = valid_row ? (ref_set ? kRescaleSlack : -INFINITY) : INFINITY;
            l *= alpha;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
#pragma unroll
            for (int r = 0; r < 16; ++r) xc[r] -= shift;
        }
    };

    // slot 0: wait for its K copy, scores, first reference
    wait_vmcnt<(RK + RV - 2) * NI>();
    lds_barrier();
    wait_lgkmcnt0();
    int cvk = hv[LAG];  // valid keys of the block of slot t+1
    if (active) {
        f32x16_t s = scores(KB[0]);
        const int nv0 = cvk - ks * kSubKeys;
        if (nv0 < kSubKeys) mask(s, nv0);
        logits_scale(s);
        logits_check();
    }

    // Iteration t (K = t % U): the body reads K slot t+1 from buffer
    // (K+1) % RK and V slot t from buffer K % RV; V slot t+RV-1 refills V
    // buffer (K+RV-1) % RV and K slot t+RK refills K buffer K % RK.  Returns
    // false when slot t+1 does not exist; slot t is then finished by the
    // tail.
    // One iteration's math, in fenced segments so that each matrix
    // instruction is issued beside vector work that does not depend on it:
    //   phase A  KK segments, each: K fragment read three ahead, two V reads,
    //            one S(t+1) MFMA, a share of slot t's exponentials (list A);
    //   phase B  KK segments, each: one PV(t) MFMA and a share of list B
    //            (second half of P(t) to bf16, the row sum of P(t), slot
    //            t+1's logits and running maximum).
    // Between the phases, keys >= nv of slot t+1 are masked (a rare,
    // wave-uniform branch: only a block's last, partly valid sub-tiles).
    auto body = [&](const uint16_t* kbuf, const uint16_t* vbuf, int nv) __attribute__((always_inline)) {
        constexpr int KD = KS == 2 ? 2 : 3;         // K fragment read distance (registers)
        constexpr int VPS = 4 * DT / KK;            // V reads per phase-A segment
        constexpr int NA = 16 + 4;                  // list A: 16 exp2, 4 packs of P[0..7]
        constexpr int NB = 4 + 16 + 24;              // list B
        const char* kb = reinterpret_cast<const char*>(kbuf);
        bf16x8_t kf[KK];
        s16x4_t vr[2][DT][2];
        float p[16];
        bf16x8_t pf[2];
        f32x16_t sn;
        float m3 = -INFINITY, ls;
        auto rdk = [&](int kk) __attribute__((always_inline)) {
            kf[kk] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(kb + koff[kk]));
        };
        auto rdv = [&](int idx) __attribute__((always_inline)) {
            const int s2 = idx / (2 * DT), dt = (idx / 2) % DT, h4 = idx % 2;
            vr[s2][dt][h4] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_s16x4_t*)((__attribute__((address_space(3))) char*)vbuf + voff[dt][h4] + s2 * 16 * D * 2));
        };
        // list A: exp2 of keys 0..7, pack them, exp2 of keys 8..15
        auto opA = [&](auto I_) __attribute__((always_inline)) {
            constexpr int I = decltype(I_)::value;
            if constexpr (I < 8) {
                p[I] = __builtin_amdgcn_exp2f(xc[I]);
            } else if constexpr (I < 12) {
                constexpr int e = 2 * (I - 8);
                pf[0][e] = (__bf16)p[e];
                pf[0][e + 1] = (__bf16)p[e + 1];
            } else {
                p[I - 4] = __builtin_amdgcn_exp2f(xc[I - 4]);
            }
        };
        // list B: pack keys 8..15, row sum, logits + maximum
        auto opB = [&](auto I_) __attribute__((always_inline)) {
            constexpr int I = decltype(I_)::value;
            if constexpr (I < 4) {
                constexpr int e = 2 * I;
                pf[1][e] = (__bf16)p[8 + e];
                pf[1][e + 1] = (__bf16)p[9 + e];
            } else if constexpr (I == 4) {
                ls = p[0];
            } else if constexpr (I < 20) {
                ls += p[I - 4];
            } else {
                constexpr int q = I - 20, k = q / 3;
                if constexpr (q % 3 == 0) {
                    xc[2 * k] = fmaf(sn[2 * k], c2, -ref);
                } else if constexpr (q % 3 == 1) {
                    xc[2 * k + 1] = fmaf(sn[2 * k + 1], c2, -ref);
                } else {
                    m3 = max3_raw(m3, xc[2 * k], xc[2 * k + 1]);
                }
            }
        };
#pragma unroll
        for (int r = 0; r < 16; ++r) sn[r] = 0.f;
        // phase A (a few exponentials first, to cover the first K read)
        __builtin_amdgcn_s_setprio(0);
        constexpr int NA0 = 4;
#pragma unroll
        for (int n = 0; n < KD; ++n) rdk(n);
        static_for<0, NA0>(opA);
        sched_fence();
        static_for<0, KK>([&](auto N_) __attribute__((always_inline)) {
            constexpr int n = decltype(N_)::value;
            if constexpr (n + KD < KK) rdk(n + KD);
#pragma unroll
            for (int v = 0; v < VPS; ++v) rdv(n * VPS + v);
            sn = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[n], qf[n], sn, 0, 0, 0);
            static_for<NA0 + n * (NA - NA0) / KK, NA0 + (n + 1) * (NA - NA0) / KK>(opA);
            sched_fence();
        });
        // keep phase A's results here: without these uses the compiler sinks
        // the exponentials past the branch below, out of phase A
        __asm__ volatile("" ::"v"(p[0]), "v"(p[1]), "v"(p[2]), "v"(p[3]), "v"(p[4]), "v"(p[5]), "v"(p[6]),
                         "v"(p[7]), "v"(p[8]), "v"(p[9]), "v"(p[10]), "v"(p[11]), "v"(p[12]), "v"(p[13]),
                         "v"(p[14]), "v"(p[15]));
        __asm__ volatile("" ::"v"(pf[0]));
        if (nv < kSubKeys) mask(sn, nv);
        // phase B at a raised issue priority, kept through the end of the
        // iteration (the workgroup barrier and the next copies) until phase A:
        // the wave that is finishing its stage issues first, so the barrier
        // every wave of the workgroup waits at is reached sooner (the sparse
        // and dense launches take 3-6 % less time, A/B in one process; the
        // priority within phase A or only across the barrier gains nothing)
        __builtin_amdgcn_s_setprio(2);
        static_for<0, KK>([&](auto N_) __attribute__((always_inline)) {
            constexpr int n = decltype(N_)::value;
            constexpr int s2 = n / DT, dt = n % DT;
            const bf16x8_t vf = __builtin_bit_cast(
                bf16x8_t, __builtin_shufflevector(vr[s2][dt][0], vr[s2][dt][1], 0, 1, 2, 3, 4, 5, 6, 7));
            o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[s2], o[dt], 0, 0, 0);
            static_for<n * NB / KK, (n + 1) * NB / KK>(opB);
            sched_fence();
        });
        __asm__ volatile("" ::"v"(ls), "v"(m3));
        l += ls;
        m3l = m3;
        logits_check();
    };
    // Copies still in flight when iteration t starts: those issued after
    // the later of K slot t+1 (second copy of iteration t+1-RK) and V slot
    // t (first copy of iteration t+1-RV); the prologue's order keeps the
    // first iterations within the same count.
    constexpr int kLastK = 2 * (1 - RK) + 1, kLastV = 2 * (1 - RV);
    constexpr int kInFlight = -1 - (kLastK > kLastV ? kLastK : kLastV);
    auto tail = [&](auto K_) __attribute__((always_inline)) {
        constexpr int K = decltype(K_)::value;
        if (active) {
            s16x4_t vr[2][DT][2];
            load_v(VB[K % RV], vr);
            bf16x8_t pf[2];
            exp_p(pf);
            pv(vr, pf);
        }
    };
    auto step = [&](auto K_) __attribute__((always_inline)) -> bool {
        constexpr int K = decltype(K_)::value;
        constexpr int SUB_K = (K + RK) % SUBS, SUB_V = (K + RV - 1) % SUBS, SUB_N = (K + 1) % SUBS;
        wait_vmcnt<kInFlight * NI>();
        lds_barrier();
        wait_lgkmcnt0();  // the list prefetches of the previous iteration
        if (SUB_V == 0) {  // V's new block: VLAG blocks behind the K-copy cursor
            jv = hj[VLAG];
            vvk = hv[VLAG] < 0 ? 0 : hv[VLAG];
        }
        issue_v((K + RV - 1) % RV, SUB_V);
        if (SUB_K == 0) k_advance();
        issue_k(K % RK, SUB_K);
        if (SUB_N == 0) {
            cvk = hv[LAG];
            if (cvk < 0) {
                tail(K_);
                return false;
            }
        }
        if (active)
            body(KB[(K + 1) % RK], VB[K % RV], cvk - SUB_N * SLOTK - ks * kSubKeys);
        // the next block's list entry: two loads, on the two iterations
        // after the K-copy cursor moved (both on that one with one slot per
        // block, where the reader keeps the indices a further entry ahead)
        if constexpr (SUBS == 1) {
            list.prefetch_both();
        } else {
            if (SUB_K == 0) list.prefetch1();
            if ((K + RK - 1) % SUBS == 0) list.prefetch2();
        }
        return true;
    };
    while (static_all<0, U>(step)) {
    }
    wait_vmcnt<0>();  // the copies past the end must land before the LDS is released

    if constexpr (KS == 2) {
        // The two key shares of each query tile meet: the second wave's
        // (reference, row sums, O) go through LDS (the ring, now free: O of
        // query tile w into K buffer w, its sums and reference into V buffer
        // w) and the first wave rescales both to the larger reference.  A
        // reference never set (no valid key seen) counts as -inf: its O and
        // sums are exact zeros.
        static_assert(NWQ == 2 && RV >= 2 && DT * 16 * 64 * 4 <= SUBE * 2, "merge buffers");
        const bool w0 = wave % NWQ == 0;
        float* xo = reinterpret_cast<float*>(w0 ? KB[0] : KB[1]);
        float* xs = reinterpret_cast<float*>(w0 ? VB[0] : VB[1]);
        __syncthreads();  // every wave's ring reads are done
        if (ks == 1) {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) xo[(dt * 16 + r) * 64 + lane] = o[dt][r];
            xs[lane] = l;
            xs[64 + lane] = ref_set ? ref : -INFINITY;
        }
        __syncthreads();
        if (ks == 1) return;
        const float r1 = ref_set ? ref : -INFINITY, r2 = xs[64 + lane];
        const float mr = fmaxf(r1, r2);
        if (mr > -INFINITY) {
            const float a1 = __builtin_amdgcn_exp2f(r1 - mr), a2 = __builtin_amdgcn_exp2f(r2 - mr);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) o[dt][r] = o[dt][r] * a1 + xo[(dt * 16 + r) * 64 + lane] * a2;
            l = l * a1 + xs[lane] * a2;
            ref = mr;
        }
    }

    // epilogue
    const float lt = add_halves(l);
    const int qrow = q0 + l32;
    const bool live = active && valid_row && lt > 0.f;
    const float inv = live ? 1.f / lt : 0.f;
    uint16_t* Orow = out_row<uint16_t>(a, h, (int64_t)i * BLK + qrow, D);
    if (Orow) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int dv = dt * 32 + 8 * g + 4 * hi;
                __bf16 v4[4];
#pragma unroll
                for (int c = 0; c < 4; ++c) v4[c] = live ? (__bf16)(o[dt][4 * g + c] * inv) : (__bf16)0.f;
                uint2 packed;
                packed.x = (uint32_t)__builtin_bit_cast(uint16_t, v4[0]) |
                           ((uint32_t)__builtin_bit_cast(uint16_t, v4[1]) << 16);
                packed.y = (uint32_t)__builtin_bit_cast(uint16_t, v4[2]) |
                           ((uint32_t)__builtin_bit_cast(uint16_t, v4[3]) << 16);
                *reinterpret_cast<uint2*>(Orow + dv) = packed;
            }
    }
    if (a.lse && hi == 0)
        a.lse[(int64_t)h * a.nqb * BLK + (int64_t)i * BLK + qrow] = live ? (ref + log2f(lt)) * kLn2 : -INFINITY;
}

// fp32 path: D/32 threads per query row, each owning 32 channels of q and
// o; one key at a time with an online softmax.  A correctness path for
// fp32 inputs.
template <int BLK, int D, bool DENSE>
__global__ void __launch_bounds__(BLK * (D / 32)) attn_f32_kernel(AttnArgs a) {
    constexpr int TPQ = D / 32;
    constexpr int NT = BLK * TPQ;
    __shared__ __attribute__((aligned(16))) float Kt[BLK * D];
    __shared__ __attribute__((aligned(16))) float Vt[BLK * D];
    const int tid = threadIdx.x, qi = tid / TPQ, part = tid % TPQ;
    int h, i;
    map_item(a.heads * a.nqb, a.nqb, h, i);
    int vq = a.q_len ? a.q_len[i] : BLK;
    vq = vq < 0 ? 0 : (vq > BLK ? BLK : vq);
    const float* qrow = in_row<float>(a, h, (int64_t)i * BLK + qi, D);
    float q[32], o[32];
#pragma unroll
    for (int c = 0; c < 32; ++c) {
        q[c] = qrow ? qrow[part * 32 + c] : 0.f;
        o[c] = 0.f;
    }
    float m = -INFINITY, l = 0.f;
    int e0, e1;
    if (DENSE) {
        e0 = 0;
        e1 = a.nkb;
    } else {
        const int row = h * a.nqb + i;
        e0 = a.row_ptr[row];
        e1 = a.row_ptr[row + 1];
        e0 = e0 < 0 ? 0 : e0;
        e1 = e1 > a.col_len ? (int)a.col_len : e1;
    }
    const float* Kh = static_cast<const float*>(a.k) + h * a.k_hs;
    const float* Vh = static_cast<const float*>(a.v) + h * a.v_hs;
    for (int e = e0; e < e1; ++e) {
        const int j = DENSE ? e : a.col_idx[e];
        if (j < 0 || j >= a.nkb) continue;
        int vk = a.kv_len ? a.kv_len[j] : BLK;
        vk = vk > BLK ? BLK : vk;
        if (vk <= 0) continue;
        __syncthreads();
        const float4* ks = reinterpret_cast<const float4*>(Kh + (int64_t)j * BLK * D);
        const float4* vs = reinterpret_cast<const float4*>(Vh + (int64_t)j * BLK * D);
        for (int x = tid; x < BLK * D / 4; x += NT) {
            reinterpret_cast<float4*>(Kt)[x] = ks[x];
            reinterpret_cast<float4*>(Vt)[x] = vs[x];
        }
        __syncthreads();
        for (int u = 0; u < vk; ++u) {
            const float* kp = Kt + u * D + part * 32;
            float sp = 0.f;
#pragma unroll
            for (int c = 0; c < 32; ++c) sp = fmaf(q[c], kp[c], sp);
#pragma unroll
            for (int off = 1; off < TPQ; off <<= 1) sp += __shfl_xor(sp, off);
            const float sc = sp * a.scale;
            const float mn = fmaxf(m, sc);
            const float alpha = expf(m - mn);
            const float p = expf(sc - mn);
            l = l * alpha + p;
            const float* vp = Vt + u * D + part * 32;
#pragma unroll
            for (int c = 0; c < 32; ++c) o[c] = fmaf(p, vp[c], o[c] * alpha);
            m = mn;
        }
    }
    const bool live = qi < vq && l > 0.f;
    const float inv = live ? 1.f / l : 0.f;
    float* orow = out_row<float>(a, h, (int64_t)i * BLK + qi, D);
    if (orow)
#pragma unroll
        for (int c = 0; c < 32; ++c) orow[part * 32 + c] = live ? o[c] * inv : 0.f;
    if (a.lse && part == 0)
        a.lse[(int64_t)h * a.nqb * BLK + (int64_t)i * BLK + qi] = live ? m + logf(l) : -INFINITY;
}

template <int BLK, int D>
hipError_t launch_typed(const AttnArgs& args, int dtype, bool dense, int total, hipStream_t stream) {
    if (dtype == BSA_BF16) {
        if (dense)
            hipLaunchKernelGGL((attn_bf16_kernel<BLK, D, true>), dim3(total), dim3(BLK * 2 * attn_key_split(BLK, D)), 0,
                               stream, args);
        else
            hipLaunchKernelGGL((attn_bf16_kernel<BLK, D, false>), dim3(total), dim3(BLK * 2 * attn_key_split(BLK, D)),
                               0, stream, args);
    } else {
        if (dense)
            hipLaunchKernelGGL((attn_f32_kernel<BLK, D, true>), dim3(total), dim3(BLK * (D / 32)), 0, stream, args);
        else
            hipLaunchKernelGGL((attn_f32_kernel<BLK, D, false>), dim3(total), dim3(BLK * (D / 32)), 0, stream, args);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attn(const AttnProblem& p, bool dense, hipStream_t stream) {
    AttnArgs a;
    a.q = p.q;
    a.k = p.k;
    a.v = p.v;
    a.o = p.o;
    a.lse = p.lse;
    a.heads = p.heads;
    a.nqb = p.nqb;
    a.nkb = p.nkb;
    a.q_hs = p.q_hs;
    a.k_hs = p.k_hs;
    a.v_hs = p.v_hs;
    a.o_hs = p.o_hs;
    a.q_len = p.q_len;
    a.kv_len = p.kv_len;
    a.row_ptr = p.row_ptr;
    a.col_idx = p.col_idx;
    a.col_len = p.col_len;
    a.scale = p.scale;
    a.scale_log2 = p.scale * 1.44269504088896340736f;
    a.o_map = p.o_map;
    a.o_map_len = p.o_map_len;
    a.o_ts = p.o_ts;
    a.q_map = p.q_map;
    a.q_map_len = p.q_map_len;
    a.q_ts = p.q_ts;
    const int total = p.heads * p.nqb;
    if (p.block == 128 && p.d == 128) return launch_typed<128, 128>(a, p.dtype, dense, total, stream);
    if (p.block == 128 && p.d == 64) return launch_typed<128, 64>(a, p.dtype, dense, total, stream);
    if (p.block == 64 && p.d == 128) return launch_typed<64, 128>(a, p.dtype, dense, total, stream);
    return launch_typed<64, 64>(a, p.dtype, dense, total, stream);
}

}  // namespace bsa
