// afd_clock.hip -- device clock stamps for timing work inside captured HIP
// graphs.  Not part of the dispatch/combine library: the benchmark links it
// to bracket the rounds it times with stamps taken on the GPU itself, since
// timing events cannot be recorded inside a captured graph and an event
// pair around a graph launch also measures the launch's own fixed cost.
//
//   afd_clock_stamp(dst, stream): enqueue one single-wavefront kernel that
//     writes the GPU's constant-rate real-time counter (s_memrealtime) to
//     the device word *dst when it runs.  Capturable.  Returns 0, or 1 when
//     the launch fails.
//   afd_clock_hz(hz): the counter's rate in Hz for the current device
//     (the wall-clock rate attribute).  Returns 0, or 1 on failure.

#include <hip/hip_runtime.h>

namespace {

__global__ __launch_bounds__(64) void k_clock(unsigned long long *dst)
{
    const unsigned long long t = __builtin_amdgcn_s_memrealtime();
    // the lane index keeps the address in a vector register: a vector store
    if (threadIdx.x == 0) dst[threadIdx.x] = t;
}

}  // namespace

extern "C" int afd_clock_stamp(unsigned long long *dst, void *stream)
{
    hipLaunchKernelGGL(k_clock, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream), dst);
    return hipGetLastError() == hipSuccess ? 0 : 1;
}

extern "C" int afd_clock_hz(long long *hz)
{
    int dev = 0, khz = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 1;
    if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess || khz <= 0) return 1;
    *hz = static_cast<long long>(khz) * 1000;
    return 0;
}
