// Host build of the library's per-index Gilbert descent, for CPU tests:
// prints perm[i] (raster index of curve cell i) for a T x H x W grid.
#include <cstdio>
#include <cstdlib>

#include "gilbert_curve.h"

int main(int argc, char** argv) {
    if (argc != 4) return 2;
    const int T = atoi(argv[1]), H = atoi(argv[2]), W = atoi(argv[3]);
    const long n = (long)T * H * W;
    for (long i = 0; i < n; ++i) {
        const bsa::curve::V3 c = bsa::curve::gilbert_cell(T, H, W, i);
        printf("%ld\n", ((long)c.t * H + c.h) * W + c.w);
    }
    return 0;
}
