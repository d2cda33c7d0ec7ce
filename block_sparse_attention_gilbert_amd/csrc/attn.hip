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

// LDS tile layout: rows of D bf16 (no padding), 16-byte chunks XOR-swizzled
// by row so that the 32 rows an MFMA operand read touches fall in distinct
// banks.  Byte offset of (row, 16-byte chunk c) inside a tile.
template <int D>
__device__ __forceinline__ int tile_off(int row, int c) {
    constexpr int CPR = D / 8;  // chunks per row
    return row * (D * 2) + ((c ^ (row & (CPR - 1))) << 4);
}

// Direct global -> LDS copy of one BLK x D bf16 tile into the swizzled
// layout.  One 16-byte load per lane lands at lds_base + 16 * lane, so lane
// l of wave-instruction I fills row r = I * RPI + l / CPR, physical chunk
// l % CPR, and fetches the logical chunk that belongs there.
template <int BLK, int D, int NW>
__device__ __forceinline__ void dma_tile(const uint16_t* __restrict__ g, uint16_t* lds_tile, int wave, int lane) {
    constexpr int CPR = D / 8;
    constexpr int RPI = 64 / CPR;                  // rows per wave-instruction (1 KB)
    constexpr int NI = BLK * D * 2 / 1024 / NW;    // instructions per wave
#pragma unroll
    for (int n = 0; n < NI; ++n) {
        const int I = n * NW + wave;
        const int row = I * RPI + lane / CPR;
        const int pc = lane % CPR;
        const int c = pc ^ (row & (CPR - 1));
        const uint16_t* src = g + row * D + c * 8;
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(src),
                                         (__attribute__((address_space(3))) void*)((lds_u16_t*)lds_tile + I * 512),
                                         16, 0, 0);
    }
}

// Transposing LDS read of V: in each 16-lane group, lane i returns
// V[kb + j][dv0 + i] for j = 0..3 (four consecutive keys of one channel);
// lane a = 4j + r of the group addresses V[kb + j][dv0 + 4r .. 4r+3].
template <int D>
__device__ __forceinline__ s16x4_t v_tr_read(const uint16_t* v_tile, int kb, int dv0, int i) {
    const int j = i >> 2, r = i & 3;
    const int row = kb + j;
    const int col = dv0 + 4 * r;  // 4-element piece: chunk col/8, half (col/4)%2
    const int off = tile_off<D>(row, col >> 3) + ((col >> 2) & 1) * 8;
    lds_s16x4_t* p = (lds_s16x4_t*)((__attribute__((address_space(3))) char*)v_tile + off);
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(p);
}

template <int BLK, int D, bool DENSE>
__global__ void __launch_bounds__(BLK * 2) attn_bf16_kernel(AttnArgs a) {
    constexpr int NW = BLK / 32;           // waves; each owns 32 query rows
    constexpr int KT = BLK / 32, DT = D / 32, KK = D / 16;
    constexpr int TILE = BLK * D;          // elements per K or V tile
    // two stages of (K tile, V tile)
    __shared__ __attribute__((aligned(1024))) uint16_t lds[2 * 2 * TILE];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int hi = lane >> 5, l32 = lane & 31, g16 = lane & 15;
    int h, i;
    map_item(a.heads * a.nqb, a.nqb, h, i);
    int vq = a.q_len ? a.q_len[i] : BLK;
    vq = vq < 0 ? 0 : (vq > BLK ? BLK : vq);
    const int q0 = wave * 32;
    const bool active = q0 < vq;

    const uint16_t* Qb = static_cast<const uint16_t*>(a.q) + h * a.q_hs + (int64_t)i * BLK * D;
    const uint16_t* Kh = static_cast<const uint16_t*>(a.k) + h * a.k_hs;
    const uint16_t* Vh = static_cast<const uint16_t*>(a.v) + h * a.v_hs;

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
    // next listed block at or after e with at least one valid key, or -1
    auto next_valid = [&](int& e, int& j, int& vk) {
        for (; e < e1; ++e) {
            j = DENSE ? e : a.col_idx[e];
            if (j < 0 || j >= a.nkb) continue;
            vk = a.kv_len ? a.kv_len[j] : BLK;
            vk = vk > BLK ? BLK : vk;
            if (vk > 0) return true;
        }
        return false;
    };

    int e = e0, j = 0, vk = 0;
    bool have = next_valid(e, j, vk);
    if (have) {
        dma_tile<BLK, D, NW>(Kh + (int64_t)j * TILE, lds, wave, lane);
        dma_tile<BLK, D, NW>(Vh + (int64_t)j * TILE, lds + TILE, wave, lane);
    }

    bf16x8_t qf[KK];
    {
        const uint16_t* qrow = Qb + (int64_t)(q0 + l32) * D + 8 * hi;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) qf[kk] = lds_bf16x8(qrow + 16 * kk);
    }
    f32x16_t o[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;
    float m = -INFINITY, l = 0.f;
    const int kr = key_of_row(l32);
    int stage = 0;

    while (have) {
        // this stage's tile has landed (every wave waited on its own copies)
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        const int vk_cur = vk;
        int en = e + 1, jn = 0, vkn = 0;
        const bool have_next = next_valid(en, jn, vkn);
        if (have_next) {
            uint16_t* nxt = lds + (stage ^ 1) * 2 * TILE;
            dma_tile<BLK, D, NW>(Kh + (int64_t)jn * TILE, nxt, wave, lane);
            dma_tile<BLK, D, NW>(Vh + (int64_t)jn * TILE, nxt + TILE, wave, lane);
        }
        const uint16_t* Kt = lds + stage * 2 * TILE;
        const uint16_t* Vt = Kt + TILE;

        if (active) {
            // S^T = K Q^T: lane holds scores of query q0 + l32 for keys
            // mt*32 + 16*(r/8) + 8*hi + (r%8), r = 0..15.
            f32x16_t s[KT];
#pragma unroll
            for (int mt = 0; mt < KT; ++mt) {
#pragma unroll
                for (int r = 0; r < 16; ++r) s[mt][r] = 0.f;
                const int key = mt * 32 + kr;
#pragma unroll
                for (int kk = 0; kk < KK; ++kk) {
                    const bf16x8_t kf = __builtin_bit_cast(
                        bf16x8_t, *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(Kt) +
                                                                   tile_off<D>(key, 2 * kk + hi)));
                    s[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[kk], s[mt], 0, 0, 0);
                }
            }
            if (vk_cur < BLK) {
#pragma unroll
                for (int mt = 0; mt < KT; ++mt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = mt * 32 + 16 * (r >> 3) + 8 * hi + (r & 7);
                        if (key >= vk_cur) s[mt][r] = -INFINITY;
                    }
            }
            float mx = -INFINITY;
#pragma unroll
            for (int mt = 0; mt < KT; ++mt)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[mt][r]);
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float mn = fmaxf(m, mx * a.scale_log2);
            const float alpha = exp2f(m - mn);
            m = mn;
            float ls = 0.f;
            bf16x8_t pf[KT][2];
#pragma unroll
            for (int mt = 0; mt < KT; ++mt)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float p = exp2f(fmaf(s[mt][r], a.scale_log2, -mn));
                    ls += p;
                    pf[mt][r >> 3][r & 7] = (__bf16)p;
                }
            l = l * alpha + ls;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;

            // O^T += V^T P^T: A = V^T fragment (8 consecutive keys of channel
            // dt*32 + l32) from two transposing reads; B = P^T from registers.
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const int dv0 = dt * 32 + 16 * ((lane >> 4) & 1);
#pragma unroll
                for (int mt = 0; mt < KT; ++mt)
#pragma unroll
                    for (int s2 = 0; s2 < 2; ++s2) {
                        const int kb = mt * 32 + 16 * s2 + 8 * hi;
                        const s16x4_t v0 = v_tr_read<D>(Vt, kb, dv0, g16);
                        const s16x4_t v1 = v_tr_read<D>(Vt, kb + 4, dv0, g16);
                        const bf16x8_t vf = __builtin_bit_cast(
                            bf16x8_t, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
                        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[mt][s2], o[dt], 0, 0, 0);
                    }
            }
        }
        stage ^= 1;
        e = en;
        j = jn;
        vk = vkn;
        have = have_next;
    }

    // epilogue
    const float lt = l + __shfl_xor(l, 32);
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
