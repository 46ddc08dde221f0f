// Shader-clock probe: a measurement utility beside the attention kernels.
//
// One wave records pairs (shader-clock counter, 100 MHz real-time counter)
// at intervals while other kernels run on other streams; the ratio of their
// advances over an interval is the shader clock during it. Timing a kernel
// with events gives seconds; this gives the clock those seconds ran at, so a
// kernel's fraction of its peak can be stated both against the published
// clock and against the measured one.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa.h"
#include "fa_measure.h"

namespace {

constexpr int kMaxSamples = 1 << 20;

__global__ void __launch_bounds__(64) clock_probe_kernel(uint64_t* __restrict__ out, int n,
                                                        int sleep_units) {
    for (int i = 0; i < n; ++i) {
        const uint64_t t = __builtin_amdgcn_s_memtime();
        const uint64_t r = __builtin_amdgcn_s_memrealtime();
        if (threadIdx.x == 0) {
            out[2 * i] = t;
            out[2 * i + 1] = r;
        }
        // s_sleep takes an immediate: the delay is sleep_units x 127 x 64
        // clocks, spent in a loop of the largest single sleep.
        for (int s = 0; s < sleep_units; ++s) __builtin_amdgcn_s_sleep(127);
    }
}

}  // namespace

extern "C" {

fa_status_t fa_clock_probe(uint64_t* samples, int n, int sleep_units, hipStream_t stream) {
    if (n < 0 || sleep_units < 0) return FA_ERR_INVALID_ARG;
    if (n == 0) return FA_OK;
    if (!samples) return FA_ERR_INVALID_ARG;
    if (((uintptr_t)samples & 15) != 0) return FA_ERR_UNSUPPORTED;
    if (n > kMaxSamples || sleep_units > 1024) return FA_ERR_UNSUPPORTED;
    hipLaunchKernelGGL(clock_probe_kernel, dim3(1), dim3(64), 0, stream, samples, n, sleep_units);
    return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // extern "C"
