// fa_unit.hip -- test-only kernels that exercise device helpers of the library
// in isolation (built into tests/kernels/libfa_unit.so; not part of libfa).
//
// fa_unit_lane_reduce: one wavefront holds a 32 x 64 score block in the
// forward kernel's S^T accumulator layout (lane l: query l % 32, keys
// 32*kt + 8*(i/4) + 4*(l/32) + i%4 for tile kt and element i), reduces its 32
// values in-lane and combines the two half-waves with lane_pair_max and
// lane_pair_sum, as the forward kernel's softmax does.  out[2*l] is the row
// maximum lane l ends with, out[2*l + 1] the row sum.
#include <hip/hip_runtime.h>

#include "../../flashattention_forward_fa_amd/csrc/fa_device.h"

namespace {

__global__ __launch_bounds__(64) void lane_reduce_kernel(const float *S, float *out) {
    const int lane = threadIdx.x & 63;
    const int lq = lane & 31, g = lane >> 5;
    float mx = -INFINITY, sum = 0.f;
    for (int kt = 0; kt < 2; ++kt)
        for (int i = 0; i < 16; ++i) {
            const float x = S[lq * 64 + 32 * kt + 8 * (i >> 2) + 4 * g + (i & 3)];
            mx = fmaxf(mx, x);
            sum += x;
        }
    out[2 * lane] = fa::lane_pair_max(mx);
    out[2 * lane + 1] = fa::lane_pair_sum(sum);
}

}  // namespace

extern "C" int fa_unit_lane_reduce(const float *S, float *out, void *stream) {
    if (!S || !out) return -1;
    hipLaunchKernelGGL(lane_reduce_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream, S, out);
    return (int)hipGetLastError();
}
