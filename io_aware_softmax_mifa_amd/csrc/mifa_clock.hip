// mifa_clock.hip -- engine-clock probe for measurement: how fast the shader clock ran while
// other work occupied the GPU.
//
// Roofline fractions of a compute-bound kernel are quoted against the chip's peak at its
// nominal 2.4 GHz engine clock; under sustained MFMA load the clock runs lower, and the
// fraction of the peak at the clock actually sustained says how much of the gap is the
// kernel's.  The driver's reported clock is refreshed too rarely to sample it under load,
// so this probe measures it on the GPU itself: each probe wave reads the shader-clock
// counter (s_memtime, one count per engine-clock cycle) and the fixed-rate real-time
// counter (s_memrealtime) at its start and its end, sleeping in between, and the ratio of
// the two differences times the real-time rate is the mean engine clock over that span.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "mifa.h"

namespace {

constexpr int kProbes = 8;  // one single-wave workgroup per XCD (workgroups go round-robin)

// out[4*w + 0..3] = {memtime at start, realtime at start, memtime at end, realtime at end}.
// The loop ends after `span` real-time ticks, or after `max_iter` sleeps of 127*64 clocks
// whichever comes first, so every wave exits even if the real-time counter were to stall.
__global__ __launch_bounds__(64) void clock_probe_kernel(long long* __restrict__ out, long long span,
                                                         int max_iter) {
  const long long t0 = (long long)__builtin_amdgcn_s_memtime();
  const long long r0 = (long long)__builtin_amdgcn_s_memrealtime();
  long long r = r0;
  for (int i = 0; i < max_iter && r - r0 < span; ++i) {
    __builtin_amdgcn_s_sleep(127);
    r = (long long)__builtin_amdgcn_s_memrealtime();
  }
  const long long t1 = (long long)__builtin_amdgcn_s_memtime();
  const long long r1 = (long long)__builtin_amdgcn_s_memrealtime();
  if (threadIdx.x == 0) {
    long long* o = out + 4 * blockIdx.x;
    o[0] = t0;
    o[1] = r0;
    o[2] = t1;
    o[3] = r1;
  }
}

}  // namespace

extern "C" __attribute__((visibility("hidden"))) void mifa_record_hip_error(int e);

extern "C" {

int mifa_clock_probe(long long* out, int64_t span_us, int* realtime_khz, void* stream) {
  if (!out || !realtime_khz) return MIFA_ERR_NULL_POINTER;
  if (span_us < 1 || span_us > 2000000) return MIFA_ERR_BAD_SHAPE;
  if ((uintptr_t)out % 8 != 0) return MIFA_ERR_MISALIGNED;
  int dev = 0, khz = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev);
  if (e == hipSuccess && khz <= 0) e = hipErrorInvalidValue;
  if (e != hipSuccess) {
    mifa_record_hip_error((int)e);
    return MIFA_ERR_HIP;
  }
  *realtime_khz = khz;
  const long long span = (long long)span_us * khz / 1000;
  // a sleep of 127*64 clocks lasts at least 3.3 us at 2.5 GHz, i.e. 330 ticks at 100 MHz
  const long long iters = span / ((long long)khz * 33 / 10000 > 0 ? (long long)khz * 33 / 10000 : 1) + 64;
  hipLaunchKernelGGL(clock_probe_kernel, dim3(kProbes), dim3(64), 0, (hipStream_t)stream, out, span,
                     (int)(iters < 0x7fffffff ? iters : 0x7fffffff));
  e = hipGetLastError();
  if (e != hipSuccess) {
    mifa_record_hip_error((int)e);
    return MIFA_ERR_HIP;
  }
  return MIFA_OK;
}

}  // extern "C"
