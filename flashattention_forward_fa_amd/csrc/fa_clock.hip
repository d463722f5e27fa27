// fa_clock.hip -- compute-unit clock probe (diagnostics, no part of attention).
//
// A throughput figure is only comparable to the matrix cores' peak at a known
// shader clock, and the clock of a busy MI355X sits below its 2.4 GHz maximum.
// One wavefront, launched beside the work being timed (on another stream),
// records pairs (shader-clock count, constant-rate count) spaced a fixed time
// apart on the constant-rate counter; the ratio of the two counts' increments
// times the constant counter's rate is the shader clock of its compute unit
// over that window.  The wave sleeps between samples and holds a few
// registers, so it leaves the compute unit to the other kernels.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_internal.h"

FA_NS_BEGIN

__global__ __launch_bounds__(64) void fa_clock_probe_kernel(uint64_t *out, int n, unsigned interval) {
    if (threadIdx.x != 0) return;
    for (int i = 0; i < n; ++i) {
        const uint64_t ref = (uint64_t)wall_clock64();
        const uint64_t sh = (uint64_t)clock64();
        out[2 * i] = sh;
        out[2 * i + 1] = ref;
        if (i + 1 == n) break;
        // Wait `interval` ticks of the constant-rate counter.  The counter
        // always advances; the iteration cap (each sleep is at least 64
        // shader cycles, i.e. far more than one tick's worth of iterations
        // at any clock) only guarantees that the loop ends.
        for (unsigned spin = 0; spin < 64u * interval + 1024u; ++spin) {
            if ((uint64_t)wall_clock64() - ref >= interval) break;
            __builtin_amdgcn_s_sleep(1);
        }
    }
}

int launch_clock_probe(uint64_t *samples, int n, unsigned interval_ticks, void *stream) {
    hipLaunchKernelGGL(fa_clock_probe_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream, samples, n,
                       interval_ticks);
    return (int)hipGetLastError();
}

FA_NS_END  // namespace fa
