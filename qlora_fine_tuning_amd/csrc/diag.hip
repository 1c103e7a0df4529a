// Diagnostics: the shader clock seen by a kernel, for the measurement harness.
//
// One workgroup of one wave reads the shader-cycle counter and the constant 100 MHz real-time
// counter, spins until the real-time counter has advanced by `ticks` (10 ns each), and reads
// both again.  The ratio of the two deltas is the average shader clock over the spin.  The
// spin ends on the real-time counter alone, so it always finishes.
#include "launch.hpp"

namespace lora {

__global__ void __launch_bounds__(64) sclk_probe_kernel(unsigned long long* out, unsigned int ticks) {
  const unsigned long long c0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  unsigned long long r1 = r0;
  while (r1 - r0 < ticks) r1 = __builtin_amdgcn_s_memrealtime();
  const unsigned long long c1 = __builtin_amdgcn_s_memtime();
  if (threadIdx.x == 0) {
    out[0] = c1 - c0;
    out[1] = r1 - r0;
  }
}

hipError_t launch_sclk_probe(unsigned long long* out, unsigned int ticks, hipStream_t s) {
  hipLaunchKernelGGL(sclk_probe_kernel, dim3(1), dim3(64), 0, s, out, ticks);
  return hipGetLastError();
}

}  // namespace lora
