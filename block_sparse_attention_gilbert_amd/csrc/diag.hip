// Diagnostic: the achievable bf16 matrix throughput of the GPU it runs on.
// Each wave keeps four independent accumulators and issues
// v_mfma_f32_32x32x16_bf16 back to back (no memory traffic in the loop), so
// the matrix pipes stay full; the sum of the accumulators is written out so
// the work is kept.  Used by the benchmark to put the attention kernel's
// matrix rate next to what the chip delivers at its current clock.
#include <hip/hip_runtime.h>

#include "kernels.h"

namespace bsa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__global__ void __launch_bounds__(256) mfma_probe_kernel(int iters, float* __restrict__ sink) {
    const int lane = threadIdx.x & 63;
    bf16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = (__bf16)(0.001f * (lane + e));
        b[e] = (__bf16)(0.002f * (lane - e));
    }
    f32x16 acc[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[u][e] = 0.0f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int u = 0; u < 4; ++u) acc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[u], 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int e = 0; e < 16; ++e) s += acc[u][e];
    sink[blockIdx.x * 256 + threadIdx.x] = s;
}

}  // namespace

hipError_t launch_mfma_probe(int workgroups, int iters, float* sink, hipStream_t stream) {
    hipLaunchKernelGGL(mfma_probe_kernel, dim3(workgroups), dim3(256), 0, stream, iters, sink);
    return hipGetLastError();
}

}  // namespace bsa
