// Shader-clock probe for the benchmark (measurement helper, built as its own
// small library libiofa_clock.so; not part of the attention library or its
// C ABI).  One wave reads the shader-cycle counter (s_memtime) and the
// 100 MHz real-time counter (s_memrealtime), sleeps in short steps until the
// real-time counter has advanced by `ticks`, and reads both again; the ratio
// of the two differences times 100 MHz is the shader clock over that window.
// Launched on a side stream while other kernels run, it reports the clock
// those kernels ran at.  The loop ends when the real-time counter passes the
// target or after a fixed number of steps, whichever comes first.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kMaxSteps = 200000;   // each step sleeps ~127 * 64 cycles

__global__ __launch_bounds__(64) void clock_probe_kernel(unsigned long long* out,
                                                         long long ticks) {
  const unsigned long long c0 = __builtin_readcyclecounter();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  unsigned long long r1 = r0;
  for (int i = 0; i < kMaxSteps && static_cast<long long>(r1 - r0) < ticks; ++i) {
    __builtin_amdgcn_s_sleep(127);
    r1 = __builtin_amdgcn_s_memrealtime();
  }
  const unsigned long long c1 = __builtin_readcyclecounter();
  r1 = __builtin_amdgcn_s_memrealtime();
  if (threadIdx.x == 0) {
    out[0] = c1 - c0;
    out[1] = r1 - r0;
  }
}

}  // namespace

// out: device array of two 64-bit counters (shader cycles, 100 MHz ticks);
// ticks: length of the window in 100 MHz ticks (> 0); stream: hipStream_t.
// Returns 0 on success, 1 on a bad argument, 2 on a launch error.
extern "C" int iofa_clock_probe(unsigned long long* out, long long ticks, void* stream) {
  if (out == nullptr || ticks <= 0) return 1;
  hipLaunchKernelGGL(clock_probe_kernel, dim3(1), dim3(64), 0,
                     static_cast<hipStream_t>(stream), out, ticks);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
