// Per-index descent of the generalized-Hilbert ("Gilbert") curve; see
// gilbert.hip for the definition.  Host and device callable.
#pragma once

#include <cstdint>

#include <hip/hip_runtime.h>

namespace bsa {
namespace curve {

struct V3 {
    int t, h, w;
};

__host__ __device__ inline int isgn(int x) { return (x > 0) - (x < 0); }
__host__ __device__ inline int vlen(V3 v) { return (v.t < 0 ? -v.t : v.t) + (v.h < 0 ? -v.h : v.h) + (v.w < 0 ? -v.w : v.w); }
__host__ __device__ inline V3 vunit(V3 v) { return {isgn(v.t), isgn(v.h), isgn(v.w)}; }
__host__ __device__ inline V3 vadd(V3 a, V3 b) { return {a.t + b.t, a.h + b.h, a.w + b.w}; }
__host__ __device__ inline V3 vsub(V3 a, V3 b) { return {a.t - b.t, a.h - b.h, a.w - b.w}; }
__host__ __device__ inline V3 vneg(V3 a) { return {-a.t, -a.h, -a.w}; }
__host__ __device__ inline V3 vmul(V3 a, int k) { return {a.t * k, a.h * k, a.w * k}; }

__host__ __device__ inline V3 even_half(V3 v) {
    const int n = vlen(v);
    int h = n / 2;
    if ((h & 1) && n > 2) ++h;
    return vmul(vunit(v), h);
}

// Cell at curve position idx of the T x H x W grid.
__host__ __device__ inline V3 gilbert_cell(int T, int H, int W, int64_t idx) {
    // axes in tie order w, h, t, stably sorted by decreasing length (a
    // three-element insertion sort written out, so nothing is indexed)
    V3 a = {0, 0, W}, b = {0, H, 0}, c = {T, 0, 0};
    if (vlen(b) > vlen(a)) {
        const V3 x = a;
        a = b;
        b = x;
    }
    if (vlen(c) > vlen(b)) {
        const V3 x = b;
        b = c;
        c = x;
        if (vlen(b) > vlen(a)) {
            const V3 y = a;
            a = b;
            b = y;
        }
    }
    V3 p = {0, 0, 0};
    // every count below is at most the grid's cell count, which the callers
    // keep below 2^31, so the descent runs in 32-bit integers
    int i = (int)idx;

    // three-dimensional levels
    for (;;) {
        const int la = vlen(a), lb = vlen(b), lc = vlen(c);
        if (lb == 1 && lc == 1) return vadd(p, vmul(vunit(a), i));
        if (lc == 1) break;  // plane (a, b)
        if (lb == 1) {       // plane (a, c)
            b = c;
            break;
        }
        if (la == 1) {  // face (b, c), travelling the longer
            if (lb >= lc) {
                a = b;
                b = c;
            } else {
                a = c;
            }
            break;
        }
        if (lb == 2 && lc == 2) {
            if (la == 2) {
                if (i < 4) {
                    a = b;
                    b = c;
                } else {
                    i -= 4;
                    p = vadd(vadd(p, vunit(a)), vsub(b, vunit(b)));
                    a = vneg(b);
                    b = c;
                }
                break;
            }
            const V3 a2 = even_half(a);
            const int n1 = vlen(a2) * 4;
            if (i < n1) {
                a = a2;
            } else {
                i -= n1;
                p = vadd(p, a2);
                a = vsub(a, a2);
            }
            continue;
        }
        if (2 * la > 3 * (lb > lc ? lb : lc)) {
            const V3 a2 = even_half(a);
            const int n1 = vlen(a2) * lb * lc;
            if (i < n1) {
                a = a2;
            } else {
                i -= n1;
                p = vadd(p, a2);
                a = vsub(a, a2);
            }
            continue;
        }
        V3 L, O;
        if (lb >= lc) {
            L = b;
            O = c;
        } else {
            L = c;
            O = b;
        }
        const V3 a2 = even_half(a), L2 = even_half(L);
        const int lL = vlen(L), lO = vlen(O), lL2 = vlen(L2), la2 = vlen(a2);
        const int n1 = lL2 * la2 * lO;
        const int n2 = la * (lL - lL2) * lO;
        if (i < n1) {
            a = L2;
            b = a2;
            c = O;
        } else if (i < n1 + n2) {
            i -= n1;
            p = vadd(p, L2);
            b = vsub(L, L2);
            c = O;
        } else {
            i -= n1 + n2;
            p = vadd(p, vadd(vsub(a, vunit(a)), vsub(L2, vunit(L))));
            const V3 na = vneg(L2), nb = vneg(vsub(a, a2));
            a = na;
            b = nb;
            c = O;
        }
    }

    // two-dimensional levels in the plane (a, b)
    for (;;) {
        const int la = vlen(a), lb = vlen(b);
        if (lb == 1) return vadd(p, vmul(vunit(a), i));
        if (la == 1) return vadd(p, vmul(vunit(b), i));
        const V3 a2 = even_half(a), b2 = even_half(b);
        if (2 * la > 3 * lb) {
            const int n1 = vlen(a2) * lb;
            if (i < n1) {
                a = a2;
            } else {
                i -= n1;
                p = vadd(p, a2);
                a = vsub(a, a2);
            }
            continue;
        }
        const int n1 = vlen(b2) * vlen(a2);
        const int n2 = la * (lb - vlen(b2));
        if (i < n1) {
            a = b2;
            b = a2;
        } else if (i < n1 + n2) {
            i -= n1;
            p = vadd(p, b2);
            b = vsub(b, b2);
        } else {
            i -= n1 + n2;
            p = vadd(p, vadd(vsub(a, vunit(a)), vsub(b2, vunit(b))));
            const V3 na = vneg(b2), nb = vneg(vsub(a, a2));
            a = na;
            b = nb;
        }
    }
}

}  // namespace curve
}  // namespace bsa
