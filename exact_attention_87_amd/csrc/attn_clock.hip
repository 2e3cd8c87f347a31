// Measurement helper: the shader clock of a running device.  Under sustained
// matrix-core load the board holds its power limit by lowering the graphics
// clock, and the clock recovers within microseconds once the load stops, so a
// reading taken between kernels says little.  This kernel is meant to run on
// a second stream beside the work being measured: each of its one-wave
// workgroups compares the shader-clock counter of the XCD it runs on with the
// 100 MHz real-time counter over a bounded spin (workgroups are dealt round
// robin to the 8 XCDs, so 8 of them sample every XCD once).  It does no
// attention arithmetic.
#include "attn_launch.h"

namespace attn {

__global__ __launch_bounds__(64) void clock_probe_kernel(unsigned long long* out, unsigned ticks) {
  const unsigned long long t0 = __builtin_amdgcn_s_memrealtime();
  const unsigned long long c0 = __builtin_amdgcn_s_memtime();
  unsigned long long t = t0;
  // Ends after `ticks` real-time ticks (at most 2 s), or after 2^23
  // iterations should the real-time counter not advance.  Each iteration
  // sleeps 640 shader cycles (0.27 us at 2.4 GHz, so the cap lies beyond 2 s
  // at any clock up to 2.4 GHz, and within 6 s at any clock above 1 GHz).
  for (int i = 0; i < (1 << 23) && t - t0 < ticks; ++i) {
    __builtin_amdgcn_s_sleep(10);
    t = __builtin_amdgcn_s_memrealtime();
  }
  const unsigned long long c1 = __builtin_amdgcn_s_memtime();
  if (threadIdx.x == 0) {
    out[2 * blockIdx.x] = c1 - c0;
    out[2 * blockIdx.x + 1] = t - t0;
  }
}

hipError_t launch_clock_probe(unsigned long long* out, int nwg, unsigned ticks, hipStream_t stream) {
  hipLaunchKernelGGL(clock_probe_kernel, dim3(nwg), dim3(64), 0, stream, out, ticks);
  return hipGetLastError();
}

}  // namespace attn
