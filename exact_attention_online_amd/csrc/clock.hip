// Clock probe: a measurement aid beside the attention kernels, not a step of the method.
//
// Under full matrix-core load the engine clock of an MI355X settles well below its 2.4 GHz peak,
// so a fraction of the spec peak mixes kernel quality with the clock.  This kernel measures the
// clock the other kernels actually ran at: each of its single-wave workgroups reads the shader
// clock counter (s_memtime, one tick per engine clock) and the constant 100 MHz real-time counter
// (s_memrealtime) at its start, sleeps in short steps until `ticks` real-time ticks have passed,
// reads both again and stores the two differences.  Launched on a second stream beside a
// workload, workgroup i starts on XCD i % 8, so 8 workgroups sample every XCD; the clock of
// workgroup i is 100 MHz * cycles / ticks.  The waves spend their time in s_sleep and take
// almost no issue slots, but each holds a wave slot and a few registers on one compute unit.
#include "common.hpp"

namespace eao {

__global__ __launch_bounds__(64) void clock_probe_kernel(unsigned long long* __restrict__ out, long long ticks) {
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  const unsigned long long c0 = __builtin_amdgcn_s_memtime();
  unsigned long long r1 = r0;
  // every wave leaves once `ticks` real-time ticks (bounded on the host) have passed
  while ((long long)(r1 - r0) < ticks) {
    __builtin_amdgcn_s_sleep(64);
    r1 = __builtin_amdgcn_s_memrealtime();
  }
  const unsigned long long c1 = __builtin_amdgcn_s_memtime();
  if (threadIdx.x == 0) {
    out[2 * blockIdx.x] = c1 - c0;
    out[2 * blockIdx.x + 1] = r1 - r0;
  }
}

hipError_t launch_clock_probe(unsigned long long* out, int groups, long long ticks, hipStream_t stream) {
  hipLaunchKernelGGL(clock_probe_kernel, dim3(groups), dim3(64), 0, stream, out, ticks);
  return hipGetLastError();
}

}  // namespace eao
