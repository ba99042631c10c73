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

// MFMA rate probe, the second measurement aid: the dense bf16 (or fp8) matrix-core rate the chip
// sustains on given operand data.  The matrix cores' power depends on the bits they multiply, and under
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

// The same for fp8 e4m3 operands (`data` as bytes): 8 A and 8 B fragments of 32 bytes per lane and
// iters x 32 back-to-back v_mfma_scale_f32_32x32x64_f8f6f4 (unit scales).
typedef __attribute__((ext_vector_type(8))) int i32x8_probe_t;

__global__ __launch_bounds__(512, 1) void mfma_probe_fp8_kernel(const uint8_t* __restrict__ data, size_t n,
                                                                 float* __restrict__ out, int iters) {
  i32x8_probe_t a[8], b[8];
  auto frag = [&](size_t at) __attribute__((always_inline)) {
    const uint4 lo = *(const uint4*)(data + at % n);
    const uint4 hi = *(const uint4*)(data + (at + 16) % n);
    return i32x8_probe_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  };
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = frag((size_t)blockIdx.x * 262144 + threadIdx.x * 512 + i * 32);
    b[i] = frag((size_t)blockIdx.x * 262144 + threadIdx.x * 512 + 256 + i * 32);
  }
  f32x16_t acc[4] = {};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[(i + j) & 7], b[i], acc[j], 0, 0, 0, 127, 0, 127);
  }
  float x = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) x += acc[j][r];
  out[(size_t)blockIdx.x * 512 + threadIdx.x] = x;
}

hipError_t launch_mfma_probe(const void* data, size_t n, bool fp8, float* out, int groups, int iters,
                             hipStream_t stream) {
  if (fp8)
    hipLaunchKernelGGL(mfma_probe_fp8_kernel, dim3(groups), dim3(512), 0, stream, (const uint8_t*)data, n, out, iters);
  else
    hipLaunchKernelGGL(mfma_probe_kernel, dim3(groups), dim3(512), 0, stream, (const uint16_t*)data, n, out, iters);
  return hipGetLastError();
}

// HBM read probe, the third measurement aid: the rate at which the chip streams device memory into
// LDS with the direct buffer -> LDS loads the kernels use, in the split-KV decoding kernel's
// pattern.  Each workgroup is one wave that streams its contiguous share of `data` in 16 KB
// stages through a ring of four LDS slots (distinct objects), requesting three stages ahead and
// waiting on its vector-memory counter for the oldest stage only; each lane adds up, modulo 2^32,
// the 32-bit words it brought in and stores the sum, so every byte is read and the result can be
// checked.
constexpr int kProbeStage = 16384;   // bytes per stage (16 direct loads of 1 KB)

template <int n>
__device__ __forceinline__ void probe_wait() {   // vmcnt n (bits 3:0 and 15:14), lgkmcnt 0
  static_assert(n >= 0 && n < 64, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(0x0070 | (n & 15) | ((n >> 4) << 14));
}

__global__ __launch_bounds__(64) void hbm_probe_kernel(const uint8_t* __restrict__ data, uint32_t share,
                                                       uint32_t* __restrict__ out) {
  __shared__ __attribute__((aligned(1024))) short ring0[kProbeStage / 2];
  __shared__ __attribute__((aligned(1024))) short ring1[kProbeStage / 2];
  __shared__ __attribute__((aligned(1024))) short ring2[kProbeStage / 2];
  __shared__ __attribute__((aligned(1024))) short ring3[kProbeStage / 2];
  auto slot = [&](auto sl) __attribute__((always_inline)) -> short* {
    constexpr int SL = decltype(sl)::value;
    if constexpr (SL == 0) return ring0;
    else if constexpr (SL == 1) return ring1;
    else if constexpr (SL == 2) return ring2;
    else return ring3;
  };
  const int lane = threadIdx.x;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(data + (size_t)blockIdx.x * share, share);
  const int nst = (int)(share / kProbeStage);
  auto issue = [&](int j, auto sl) __attribute__((always_inline)) {
    short* dst = slot(sl);
#pragma unroll
    for (int i = 0; i < 16; ++i) buffer_load16_lds(rs, dst + 512 * i, 16 * lane, (uint32_t)j * kProbeStage + 1024 * i);
  };
  uint32_t acc = 0;
  auto stage = [&](int j, auto sl) __attribute__((always_inline)) {
    constexpr int SL = decltype(sl)::value;
    const int ahead = min(2, nst - 1 - j);
    if (ahead >= 2) probe_wait<32>();
    else if (ahead == 1) probe_wait<16>();
    else probe_wait<0>();
    if (j + 3 < nst) issue(j + 3, std::integral_constant<int, (SL + 3) % 4>{});
    const short* src = slot(sl);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint4 v = *(const uint4*)(src + 512 * i + 8 * lane);
      acc += v.x + v.y + v.z + v.w;
    }
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;
  using S3 = std::integral_constant<int, 3>;
  if (nst > 0) issue(0, S0{});
  if (nst > 1) issue(1, S1{});
  if (nst > 2) issue(2, S2{});
  for (int j = 0; j < nst; j += 4) {
    stage(j, S0{});
    if (j + 1 >= nst) break;
    stage(j + 1, S1{});
    if (j + 2 >= nst) break;
    stage(j + 2, S2{});
    if (j + 3 >= nst) break;
    stage(j + 3, S3{});
  }
  out[(size_t)blockIdx.x * 64 + lane] = acc;
}

hipError_t launch_hbm_probe(const uint8_t* data, uint32_t share, uint32_t* out, int groups, hipStream_t stream) {
  hipLaunchKernelGGL(hbm_probe_kernel, dim3(groups), dim3(64), 0, stream, data, share, out);
  return hipGetLastError();
}

}  // namespace eao
