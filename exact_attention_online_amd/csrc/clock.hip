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

// MFMA rate probe, the second measurement aid: the dense bf16 matrix-core rate the chip sustains
// on given operand data.  The matrix cores' power depends on the bits they multiply, and under
// the board's power limit the engine clock follows, so random operands run well below the spec
// peak while zero operands come close to it.  Each workgroup is 8 waves (two per SIMD of a compute
// unit, as the attention kernels run); each wave loads 8 A and 8 B fragments (16 bytes per lane)
// from `data` and issues iters x 32 back-to-back v_mfma_f32_32x32x16_bf16 into four
// accumulators, then every lane stores the sum of its accumulators (so nothing is dead code).
__global__ __launch_bounds__(512, 1) void mfma_probe_kernel(const uint16_t* __restrict__ data, size_t n,
                                                             float* __restrict__ out, int iters) {
  i16x8_t a[8], b[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const size_t ia = ((size_t)blockIdx.x * 8192 + threadIdx.x * 128 + i * 8) % n;
    const size_t ib = ((size_t)blockIdx.x * 8192 + threadIdx.x * 128 + 64 + i * 8) % n;
    a[i] = __builtin_bit_cast(i16x8_t, *(const uint4*)(data + ia));
    b[i] = __builtin_bit_cast(i16x8_t, *(const uint4*)(data + ib));
  }
  f32x16_t acc[4] = {};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] = mfma32x32x16<true>(a[(i + j) & 7], b[i], acc[j]);
  }
  float x = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) x += acc[j][r];
  out[(size_t)blockIdx.x * 512 + threadIdx.x] = x;
}

hipError_t launch_mfma_probe(const uint16_t* data, size_t n, float* out, int groups, int iters, hipStream_t stream) {
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(groups), dim3(512), 0, stream, data, n, out, iters);
  return hipGetLastError();
}

}  // namespace eao
