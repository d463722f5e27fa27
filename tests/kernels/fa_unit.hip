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
//
// fa_unit_issue_rates: one 8-wave workgroup per compute unit (waves w and
// w + 4 share a SIMD).  Waves 0-3 run role_a, waves 4-7 role_b, each for
// `iters` iterations of: 4 independent v_mfma_f32_32x32x16_bf16 (role 1), 32
// independent v_fma_f32 in 16 chains (role 2), or nothing (role 0); cycles[w]
// of each workgroup is the wave's shader-clock count for the loop.  The
// forward kernel's two phases are roles 1 and 2 side by side.
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

typedef float unit_f32x16 __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(512, 1) void issue_kernel(long long *cycles, float *sink, int iters,
                                                       int role_a, int role_b) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int role = w < 4 ? role_a : role_b;
    fa::bf16x8 a, b;
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(0.001f * (lane + i));
        b[i] = (__bf16)(0.002f * (i - lane));
    }
    unit_f32x16 acc[4];
    for (int m = 0; m < 4; ++m)
        for (int i = 0; i < 16; ++i) acc[m][i] = 0.f;
    float x[16];
    for (int k = 0; k < 16; ++k) x[k] = -0.5f - 0.01f * (lane + k);
    __syncthreads();
    const long long t0 = clock64();
    if (role == 1) {
        for (int it = 0; it < iters; ++it)
#pragma unroll
            for (int m = 0; m < 4; ++m) acc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[m], 0, 0, 0);
    } else if (role == 2) {
        for (int it = 0; it < iters; ++it)
#pragma unroll
            for (int r = 0; r < 2; ++r)
#pragma unroll
                for (int k = 0; k < 16; ++k) x[k] = fmaf(x[k], 0.999f, x[(k + 1) & 15]);
    }
    const long long t1 = clock64();
    float s = 0.f;
    for (int k = 0; k < 16; ++k) s += x[k];
    for (int m = 0; m < 4; ++m)
        for (int i = 0; i < 16; ++i) s += acc[m][i];
    sink[blockIdx.x * 512 + threadIdx.x] = s;   // keeps the work
    if (lane == 0) cycles[blockIdx.x * 8 + w] = t1 - t0;
}

}  // namespace

extern "C" int fa_unit_issue_rates(long long *cycles, float *sink, int grid, int iters, int role_a,
                                   int role_b, void *stream) {
    if (!cycles || !sink || grid < 1 || iters < 1) return -1;
    hipLaunchKernelGGL(issue_kernel, dim3(grid), dim3(512), 0, (hipStream_t)stream, cycles, sink,
                       iters, role_a, role_b);
    return (int)hipGetLastError();
}

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
