// Kernel launchers of the bsa library (internal; the C ABI is in bsa.h).
// Each launcher enqueues on `stream` and returns hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>

#include "common.h"

namespace bsa {

hipError_t launch_gilbert_index(int T, int H, int W, int32_t* perm, int32_t* inv, hipStream_t stream);

hipError_t launch_gilbert_perm(const void* src, void* dst, const int32_t* perm, int L, int heads, int d,
                               int block, int64_t raster_token_stride, int64_t gilbert_head_stride,
                               int inverse, int dtype, hipStream_t stream);

hipError_t launch_route(const bsa_route_args* a, const RouteLayout& lay, void* ws, hipStream_t stream);

hipError_t launch_attn(const AttnProblem& p, bool dense, hipStream_t stream);

}  // namespace bsa
