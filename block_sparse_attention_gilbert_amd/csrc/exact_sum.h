// Exact block sums in float64 for the pooled means: a double-double (hi, lo)
// whose hi + lo is the running sum.  Each addition is split by the
// error-free two-sum transformation (Knuth, TAOCP vol. 2, 4.2.2): s + e
// equals a + b exactly.  The one rounded operation per step adds two error
// terms; if every input is an integer multiple of a unit u and the largest
// magnitude is below 2^98 u, those terms stay integer multiples of u below
// 2^53 u, so the addition is exact and hi + lo is always the exact sum.
// The last two-sum then leaves in hi the exact sum rounded once to nearest
// (ties to even), whatever the order of the additions.  For float32 inputs
// the condition holds when a column's nonzero magnitudes span less than
// 2^74.  bfloat16 inputs (8 significand bits) need no pair: a plain float64
// sum of at most 128 of them never rounds while their nonzero magnitudes
// span less than 2^39 (all partial sums are integer multiples of the finest
// value's last-bit unit below 2^53 of them), so the block sums use
// Acc<true> = a plain double there, Acc<false> = dd for float32.
#pragma once

#include <hip/hip_runtime.h>

namespace bsa {

struct dd {
    double hi, lo;
};

__device__ __forceinline__ void two_sum(double a, double b, double& s, double& e) {
    s = a + b;
    const double bb = s - a;
    e = (a - (s - bb)) + (b - bb);
}

__device__ __forceinline__ dd dd_add(dd x, double v) {
    double s, e;
    two_sum(x.hi, v, s, e);
    dd r;
    two_sum(s, x.lo + e, r.hi, r.lo);
    return r;
}

__device__ __forceinline__ dd dd_add(dd x, dd y) {
    double s, e;
    two_sum(x.hi, y.hi, s, e);
    dd r;
    two_sum(s, (x.lo + y.lo) + e, r.hi, r.lo);
    return r;
}

__device__ __forceinline__ dd dd_shfl_xor(dd x, int off) { return dd{__shfl_xor(x.hi, off), __shfl_xor(x.lo, off)}; }

// Block-sum accumulator of one column: plain float64 for bf16 inputs, a
// double-double for float32 inputs (see above).
template <bool BF16>
struct Acc;

template <>
struct Acc<true> {
    double s = 0.0;
    __device__ __forceinline__ void add(double v) { s += v; }
    __device__ __forceinline__ void add(const Acc& o) { s += o.s; }
    __device__ __forceinline__ Acc shfl_xor(int off) const {
        Acc r;
        r.s = __shfl_xor(s, off);
        return r;
    }
    __device__ __forceinline__ double hi() const { return s; }
    __device__ __forceinline__ double lo() const { return 0.0; }
    __device__ __forceinline__ static Acc make(double h, double) {
        Acc r;
        r.s = h;
        return r;
    }
};

template <>
struct Acc<false> {
    dd s{0.0, 0.0};
    __device__ __forceinline__ void add(double v) { s = dd_add(s, v); }
    __device__ __forceinline__ void add(const Acc& o) { s = dd_add(s, o.s); }
    __device__ __forceinline__ Acc shfl_xor(int off) const {
        Acc r;
        r.s = dd_shfl_xor(s, off);
        return r;
    }
    __device__ __forceinline__ double hi() const { return s.hi; }
    __device__ __forceinline__ double lo() const { return s.lo; }
    __device__ __forceinline__ static Acc make(double h, double l) {
        Acc r;
        r.s = dd{h, l};
        return r;
    }
};

}  // namespace bsa
