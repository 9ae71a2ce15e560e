// attn_clock.hip -- a measurement aid: the shader clock of one CU over a
// wall-clock interval, so that throughput can be set against the MFMA peak
// at the clock the chip actually ran (the pages compare kernels with the
// peak of their chip: "Lecture 9 -- Hopper / FlashAttention-3 /
// FlashAttention-4", "Measure it").
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace attn {

// One lane spins until the constant-rate wall clock has advanced by `ticks`
// (or a fixed iteration cap, so the wave always ends), then writes the
// shader-clock and wall-clock deltas.
__global__ void __launch_bounds__(64) clock_probe_kernel(unsigned long long* out, long long ticks) {
  if (threadIdx.x != 0) return;
  const unsigned long long r0 = wall_clock64(), c0 = clock64();
  unsigned long long r1 = r0, c1 = c0;
  for (long long i = 0; i < (1LL << 30) && (long long)(r1 - r0) < ticks; ++i) {
    r1 = wall_clock64();
    c1 = clock64();
  }
  out[0] = c1 - c0;
  out[1] = r1 - r0;
}

hipError_t launch_clock_probe(unsigned long long* out, long long ticks, hipStream_t s) {
  hipLaunchKernelGGL(clock_probe_kernel, dim3(1), dim3(64), 0, s, out, ticks);
  return hipGetLastError();
}

}  // namespace attn
