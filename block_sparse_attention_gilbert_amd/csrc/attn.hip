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
};

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
constexpr int kStages = 4;    // LDS stages; kStages - 1 sub-tiles in flight
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

// Direct global -> LDS copy of one kSubKeys x D bf16 sub-tile into the
// swizzled layout.  One 16-byte load per lane lands at base + 16 * lane, so
// lane l of wave-instruction I fills row I * RPI + l / CPR, physical chunk
// l % CPR, and fetches the logical chunk that belongs there.
template <int D, int NW, bool IS_V>
__device__ __forceinline__ void dma_sub(const uint16_t* __restrict__ g, uint16_t* lds_tile, int wave, int lane) {
    constexpr int CPR = D / 8;
    constexpr int RPI = 64 / CPR;                     // rows per wave-instruction (1 KB)
    constexpr int NI = kSubKeys * D * 2 / 1024 / NW;  // instructions per wave
#pragma unroll
    for (int n = 0; n < NI; ++n) {
        const int I = n * NW + wave;
        const int row = I * RPI + lane / CPR;
        const int c = (lane % CPR) ^ swz<D, IS_V>(row);
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(g + row * D + c * 8),
                                         (__attribute__((address_space(3))) void*)((lds_u16_t*)lds_tile + I * 512),
                                         16, 0, 0);
    }
}

// max over the two lanes l and l ^ 32 (which hold one query's two key halves)
__device__ __forceinline__ float max_halves(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float add_halves(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Workgroup barrier for the copy pipeline.  A fenced barrier
// (__syncthreads, or an LDS-scoped fence, since LDS-DMA writes are pending
// LDS writes) makes the compiler drain every outstanding copy, including the
// stages still streaming in.  Here each wave has already waited (vmcnt) for
// its own copies of the stage about to be read, and every read of the stage
// about to be overwritten was consumed by an MFMA before the barrier, so a
// bare s_barrier is enough; the empty asm statements only stop the compiler
// from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    // gfx9 s_waitcnt: vmcnt[3:0] and [15:14], expcnt[6:4] (7 = no wait),
    // lgkmcnt[11:8] (15 = no wait)
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Cursor over the listed blocks of a row: block j with vk valid keys,
// skipping out-of-range entries and blocks without valid keys.  When the
// list is exhausted `have` drops and j keeps the last valid block.
template <int BLK, bool DENSE>
struct BlockCursor {
    int e, e1, j, vk;
    bool have;
    const_i32_t* col;
    const_i32_t* kvl;
    int nkb;
    __device__ __forceinline__ void next() {
        for (; e < e1; ++e) {
            const int jj = DENSE ? e : col[e];
            if (jj < 0 || jj >= nkb) continue;
            int v = kvl ? kvl[jj] : BLK;
            v = v > BLK ? BLK : v;
            if (v > 0) {
                j = jj;
                vk = v;
                ++e;
                have = true;
                return;
            }
        }
        have = false;
    }
};

// Workgroup of BLK/32 waves, one (head, query block); wave w owns query rows
// 32w .. 32w+31 and every key.  Each 32-key stage is 2 x 8 KB (d = 128), so
// a workgroup needs 64 KB of LDS and two workgroups share a CU: their
// independent barriers let the hardware overlap one workgroup's softmax and
// LDS latency with the other's matrix instructions.
template <int BLK, int D, bool DENSE>
__global__ void __launch_bounds__(BLK * 2, 2) attn_bf16_kernel(AttnArgs a) {
    constexpr int NW = BLK / 32;               // waves
    constexpr int DT = D / 32, KK = D / 16;
    constexpr int SUBE = kSubKeys * D;         // elements of a K or V sub-tile
    constexpr int NI = 2 * (kSubKeys * D * 2 / 1024 / NW);  // DMA instructions per wave per stage
    static_assert(kSubKeys * D * 2 % (1024 * NW) == 0, "stage copy must split evenly over the waves");
    __shared__ __attribute__((aligned(1024))) uint16_t st0[2 * SUBE];
    __shared__ __attribute__((aligned(1024))) uint16_t st1[2 * SUBE];
    __shared__ __attribute__((aligned(1024))) uint16_t st2[2 * SUBE];
    __shared__ __attribute__((aligned(1024))) uint16_t st3[2 * SUBE];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int hi = lane >> 5, l32 = lane & 31, g16 = lane & 15;
    int h, i;
    map_item(a.heads * a.nqb, a.nqb, h, i);
    int vq = a.q_len ? a.q_len[i] : BLK;
    vq = vq < 0 ? 0 : (vq > BLK ? BLK : vq);
    const int q0 = wave * 32;
    const bool active = q0 < vq;
    const bool valid_row = q0 + l32 < vq;

    const uint16_t* Qb = static_cast<const uint16_t*>(a.q) + h * a.q_hs + (int64_t)i * BLK * D;
    const uint16_t* Kh = static_cast<const uint16_t*>(a.k) + h * a.k_hs;
    const uint16_t* Vh = static_cast<const uint16_t*>(a.v) + h * a.v_hs;

    // Q^T fragments (B operand of S^T = K Q^T), held for the whole walk
    bf16x8_t qf[KK];
    {
        const uint16_t* qrow = Qb + (int64_t)(q0 + l32) * D + 8 * hi;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) qf[kk] = lds_bf16x8(qrow + 16 * kk);
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
    // Every listed block is SUBS stages of kSubKeys keys; slot t is stage
    // t % 4, sub-tile t % SUBS of block t / SUBS.  Three slots are always in
    // flight: past the end of the list the copies repeat the last block
    // (never computed), so every wait is the same vmcnt.
    constexpr int SUBS = BLK / kSubKeys;
    static_assert(kStages % SUBS == 0, "stages must hold whole blocks");
    BlockCursor<BLK, DENSE> ic{e0, e1, 0, 0, false, (const_i32_t*)a.col_idx, (const_i32_t*)a.kv_len, a.nkb};
    ic.next();
    if (!ic.have) {
        // empty list: zeros and -inf, no copies in flight
        const int qrow = q0 + l32;
        uint16_t* Orow = static_cast<uint16_t*>(a.o) + h * a.o_hs + ((int64_t)i * BLK + qrow) * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int g = 0; g < 4; ++g) *reinterpret_cast<uint2*>(Orow + dt * 32 + 8 * g + 4 * hi) = make_uint2(0u, 0u);
        if (a.lse && hi == 0) a.lse[(int64_t)h * a.nqb * BLK + (int64_t)i * BLK + qrow] = -INFINITY;
        return;
    }
    BlockCursor<BLK, DENSE> cc = ic;
    auto issue = [&](uint16_t* stage, int sub) {
        const int64_t off = ((int64_t)ic.j * BLK + sub * kSubKeys) * D;
        dma_sub<D, NW, false>(Kh + off, stage, wave, lane);
        dma_sub<D, NW, true>(Vh + off, stage + SUBE, wave, lane);
    };
    // prologue: slots 0, 1, 2
    issue(st0, 0);
    if (1 % SUBS == 0) ic.next();
    issue(st1, 1 % SUBS);
    if (2 % SUBS == 0) ic.next();
    issue(st2, 2 % SUBS);

    // per-lane LDS byte offsets (loop invariant)
    const int kr = key_of_row(l32);
    int koff[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) koff[kk] = tile_off<D, false>(kr, 2 * kk + hi);
    int voff[DT][2];
    {
        const int j4 = g16 >> 2, r4 = g16 & 3, g2 = (lane >> 4) & 1;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int h4 = 0; h4 < 2; ++h4) {
                const int row = 8 * hi + 4 * h4 + j4;  // + 16*s2
                const int col = dt * 32 + 16 * g2 + 4 * r4;
                voff[dt][h4] = tile_off<D, true>(row, col >> 3) + ((col >> 2) & 1) * 8 + SUBE * 2;
            }
    }

    f32x16_t o[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;
    float m = -INFINITY, l = 0.f;
    const float c2 = a.scale_log2;

    auto compute = [&](const uint16_t* stage, int nv) {
        if (!active || nv <= 0) return;
        const char* base = reinterpret_cast<const char*>(stage);
        bf16x8_t kf[KK];
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
            kf[kk] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(base + koff[kk]));
        s16x4_t vr[2][DT][2];
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int h4 = 0; h4 < 2; ++h4)
                    vr[s2][dt][h4] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_s16x4_t*)((__attribute__((address_space(3))) char*)stage + voff[dt][h4] +
                                       s2 * 16 * D * 2));
        // S^T = K Q^T over the stage's 32 keys: lane holds the scores of
        // query q0 + l32 for keys 16*(r/8) + 8*hi + (r%8), r = 0..15.
        f32x16_t s;
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kk], qf[kk], s, 0, 0, 0);
        if (nv < kSubKeys) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = 16 * (r >> 3) + 8 * hi + (r & 7);
                if (key >= nv) s[r] = -INFINITY;
            }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
        mx = max_halves(mx) * c2;
        // lazy rescaling: a query's reference max moves only when its own
        // max passes it by more than kRescaleSlack (so p <= 2^slack); each
        // query's arithmetic depends on its own scores only.  Padded query
        // rows never move it (their results are discarded).
        const bool need = valid_row && mx > m + kRescaleSlack;
        if (__any(need)) {
            const float mn = need ? mx : m;
            const float alpha = need ? __builtin_amdgcn_exp2f(m - mn) : 1.0f;
            m = mn;
            l *= alpha;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
        }
        // padded query rows keep m = -inf: use 0 so their p stay finite
        const float mref = m == -INFINITY ? 0.f : m;
        float ls = 0.f;
        bf16x8_t pf[2];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float p = __builtin_amdgcn_exp2f(fmaf(s[r], c2, -mref));
            ls += p;
            pf[r >> 3][r & 7] = (__bf16)p;
        }
        l += ls;
        // O^T += V^T P^T; four independent chains (dt)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const bf16x8_t vf = __builtin_bit_cast(
                    bf16x8_t, __builtin_shufflevector(vr[s2][dt][0], vr[s2][dt][1], 0, 1, 2, 3, 4, 5, 6, 7));
                o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[s2], o[dt], 0, 0, 0);
            }
    };

    // Slot t (stage K = t % 4): wait for its copies, barrier, issue slot
    // t + 3 into the stage freed by slot t - 1, multiply.  Unrolled over the
    // four stages so stage arrays and sub-tile indices are compile-time.
    auto step = [&](auto K_, uint16_t* cur, uint16_t* nxt) {
        constexpr int K = decltype(K_)::value;
        constexpr int SUB_C = K % SUBS, SUB_I = (K + 3) % SUBS;
        wait_vmcnt<2 * NI>();
        lds_barrier();
        if (SUB_I == 0) ic.next();
        issue(nxt, SUB_I);
        compute(cur, cc.vk - SUB_C * kSubKeys);
        if (SUB_C == SUBS - 1) cc.next();
    };
    for (;;) {
        step(std::integral_constant<int, 0>(), st0, st3);
        if (!cc.have) break;
        step(std::integral_constant<int, 1>(), st1, st0);
        if (!cc.have) break;
        step(std::integral_constant<int, 2>(), st2, st1);
        if (!cc.have) break;
        step(std::integral_constant<int, 3>(), st3, st2);
        if (!cc.have) break;
    }
    wait_vmcnt<0>();  // the copies past the end must land before the LDS is released

    // epilogue
    const float lt = add_halves(l);
    const int qrow = q0 + l32;
    const bool live = active && qrow < vq && lt > 0.f;
    const float inv = live ? 1.f / lt : 0.f;
    uint16_t* Orow = static_cast<uint16_t*>(a.o) + h * a.o_hs + ((int64_t)i * BLK + qrow) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int dv = dt * 32 + 8 * g + 4 * hi;
            __bf16 v4[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) v4[c] = live ? (__bf16)(o[dt][4 * g + c] * inv) : (__bf16)0.f;
            uint2 packed;
            packed.x = (uint32_t)__builtin_bit_cast(uint16_t, v4[0]) | ((uint32_t)__builtin_bit_cast(uint16_t, v4[1]) << 16);
            packed.y = (uint32_t)__builtin_bit_cast(uint16_t, v4[2]) | ((uint32_t)__builtin_bit_cast(uint16_t, v4[3]) << 16);
            *reinterpret_cast<uint2*>(Orow + dv) = packed;
        }
    if (a.lse && hi == 0)
        a.lse[(int64_t)h * a.nqb * BLK + (int64_t)i * BLK + qrow] = live ? (m + log2f(lt)) * kLn2 : -INFINITY;
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
    const float* qrow = static_cast<const float*>(a.q) + h * a.q_hs + ((int64_t)i * BLK + qi) * D + part * 32;
    float q[32], o[32];
#pragma unroll
    for (int c = 0; c < 32; ++c) {
        q[c] = qrow[c];
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
    float* orow = static_cast<float*>(a.o) + h * a.o_hs + ((int64_t)i * BLK + qi) * D + part * 32;
#pragma unroll
    for (int c = 0; c < 32; ++c) orow[c] = live ? o[c] * inv : 0.f;
    if (a.lse && part == 0)
        a.lse[(int64_t)h * a.nqb * BLK + (int64_t)i * BLK + qi] = live ? m + logf(l) : -INFINITY;
}

template <int BLK, int D>
hipError_t launch_typed(const AttnArgs& args, int dtype, bool dense, int total, hipStream_t stream) {
    if (dtype == BSA_BF16) {
        if (dense)
            hipLaunchKernelGGL((attn_bf16_kernel<BLK, D, true>), dim3(total), dim3(BLK * 2), 0, stream, args);
        else
            hipLaunchKernelGGL((attn_bf16_kernel<BLK, D, false>), dim3(total), dim3(BLK * 2), 0, stream, args);
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
    const int total = p.heads * p.nqb;
    if (p.block == 128 && p.d == 128) return launch_typed<128, 128>(a, p.dtype, dense, total, stream);
    if (p.block == 128 && p.d == 64) return launch_typed<128, 64>(a, p.dtype, dense, total, stream);
    if (p.block == 64 && p.d == 128) return launch_typed<64, 128>(a, p.dtype, dense, total, stream);
    return launch_typed<64, 64>(a, p.dtype, dense, total, stream);
}

}  // namespace bsa
