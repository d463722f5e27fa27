// fa_unit.hip -- test-only kernels that exercise device helpers of the library
// in isolation (built into tests/kernels/libfa_unit.so; not part of libfa).
//
// fa_unit_lane_reduce: one wavefront holds a 32 x 64 score block in the
// forward kernel's S^T accumulator layout (lane l: query l % 32, keys
// 32*kt + 8*(i/4) + 4*(l/32) + i%4 for tile kt and element i), reduces its 32
// values in-lane and combines the two half-waves with lane_pair_max and
// lane_pair_sum, as the forward kernel's softmax does.  out[2*l] is the row
// maximum lane l ends with, out[2*l + 1] the row sum.
//
// fa_unit_xcd_of_workgroups: every workgroup of a grid of n records the XCD
// it runs on (hardware register XCC_ID) in out[workgroup index].  Workgroups of
// 512 threads with 66 KiB of LDS, one per compute unit as the d = 128 forward
// kernel's, or of 256 threads with 34 KiB, as the d = 64 forward and the
// backward kernels'.
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

template <int THREADS, int LDS_BYTES>
__global__ __launch_bounds__(THREADS) void xcd_kernel(unsigned *out) {
    __shared__ unsigned char pad[LDS_BYTES];   // the forward kernel's LDS footprint
    pad[threadIdx.x] = (unsigned char)threadIdx.x;
    __syncthreads();
    // s_getreg_b32 of HW_REG_XCC_ID (hardware register 20, bits 0..15)
    const unsigned xcc = __builtin_amdgcn_s_getreg(20 | (15 << 11)) & 0xFu;
    if (threadIdx.x == 0) out[blockIdx.x] = xcc + (pad[THREADS - 1] == (unsigned char)(THREADS - 1) ? 0u : 0x100u);
}

}  // namespace

extern "C" int fa_unit_xcd_of_workgroups(unsigned *out, int n, int big, void *stream) {
    if (!out || n < 1) return -1;
    if (big) hipLaunchKernelGGL((xcd_kernel<512, 66 * 1024>), dim3(n), dim3(512), 0, (hipStream_t)stream, out);
    else     hipLaunchKernelGGL((xcd_kernel<256, 34 * 1024>), dim3(n), dim3(256), 0, (hipStream_t)stream, out);
    return (int)hipGetLastError();
}

extern "C" int fa_unit_lane_reduce(const float *S, float *out, void *stream) {
    if (!S || !out) return -1;
    hipLaunchKernelGGL(lane_reduce_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream, S, out);
    return (int)hipGetLastError();
}
