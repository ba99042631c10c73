// Shared device helpers for the gfx950 attention kernels: MFMA wrappers, LDS swizzle and
// transpose reads, cross-half lane exchange, 16-bit conversions.
//
// Lane layouts used throughout (checked on gfx950 with a layout probe):
//   v_mfma_f32_32x32x16_{bf16,f16}:  lane l, g = l / 32
//     A operand (8 x 16-bit): A[row = l % 32][k = 8g + e], e = 0..7
//     B operand (8 x 16-bit): B[k = 8g + e][col = l % 32]
//     C/D (16 x f32):         C[row = 8(r/4) + 4g + r%4][col = l % 32], r = 0..15
//   Only the pairing of A slot (g, e) with B slot (g, e) matters for the sum over k, so any
//   consistent relabelling of k is allowed; the kernels use that to feed a C tile straight
//   back in as a B operand.
//   ds_read_b64_tr_b16: in each group of 16 lanes, lane i reads 4 x 16-bit at its own address;
//     lane j receives element (j % 4) of lanes (j / 4) + 4e, e = 0..3.  When lane i points at
//     row (i / 4), columns 4(i % 4)..4(i % 4)+3 of a 4 x 16 block, lane j receives column j.
//   v_permlane32_swap: exchanges lanes 0..31 of one operand with lanes 32..63 of the other;
//     with both operands equal, {out0, out1} = {x[l % 32], x[l % 32 + 32]} on every lane.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace eao {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;
typedef __attribute__((ext_vector_type(8))) short i16x8_t;
typedef __attribute__((ext_vector_type(4))) short i16x4_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

typedef i16x4_t __attribute__((address_space(3))) lds_i16x4_t;

constexpr float kLog2e = 1.4426950408889634f;

// Compile-time parity tags of double-buffered loops (which LDS buffer a step uses).
using Par0 = std::integral_constant<int, 0>;
using Par1 = std::integral_constant<int, 1>;
constexpr float kLn2 = 0.6931471805599453f;

// compute units of an MI355X (gfx950); grids smaller than two workgroups per unit switch to
// smaller row blocks
constexpr int kNumCUs = 256;

// C += A * B on one 32x32x16 MFMA; BF16 selects bfloat16, otherwise fp16 operands.
template <bool BF16>
__device__ __forceinline__ f32x16_t mfma32x32x16(i16x8_t a, i16x8_t b, f32x16_t c) {
  if constexpr (BF16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  }
}

// Round-to-nearest-even conversion of two floats into a packed pair of 16-bit payloads
// (one v_cvt_pk_bf16_f32 / v_cvt_pk_f16_f32).
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2_t;
template <bool BF16>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  if constexpr (BF16) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
  } else {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
  }
}

// Eight consecutive accumulator entries -> one 8 x 16-bit MFMA operand.
template <bool BF16>
__device__ __forceinline__ i16x8_t pack8(const f32x16_t& x, int base) {
  uint32_t w0 = pack2<BF16>(x[base + 0], x[base + 1]);
  uint32_t w1 = pack2<BF16>(x[base + 2], x[base + 3]);
  uint32_t w2 = pack2<BF16>(x[base + 4], x[base + 5]);
  uint32_t w3 = pack2<BF16>(x[base + 6], x[base + 7]);
  typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
  u32x4_t w = {w0, w1, w2, w3};
  return __builtin_bit_cast(i16x8_t, w);
}

template <bool BF16>
__device__ __forceinline__ float to_float(uint16_t x) {
  if constexpr (BF16) {
    return (float)__builtin_bit_cast(__bf16, x);
  } else {
    return (float)__builtin_bit_cast(_Float16, x);
  }
}

// The low / high 16-bit half of a packed pair as a float.
template <bool BF16>
__device__ __forceinline__ float lo_to_float(uint32_t pair) {
  if constexpr (BF16) {
    return __uint_as_float(pair << 16);
  } else {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(pair & 0xFFFFu));
  }
}
template <bool BF16>
__device__ __forceinline__ float hi_to_float(uint32_t pair) {
  if constexpr (BF16) {
    return __uint_as_float(pair & 0xFFFF0000u);
  } else {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(pair >> 16));
  }
}

// Larger of two scores (finite or -inf): the NaN-propagating maximum, which gfx950 does in one
// v_maximum3_f32 without first quieting its operands (fmaxf's IEEE form needs that per operand).
__device__ __forceinline__ float smax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// Row maximum of the 16 x NK scores s[0..NK-1][0..15] a lane holds (registers r and r + 4 of one
// block are the same column group): four chains, each step folding two new scores into one
// three-input maximum, then the two lane halves.
template <int NK>
__device__ __forceinline__ float row_max(const f32x16_t (&s)[NK]) {
  float mx[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    mx[e] = smax(s[0][e], s[0][e + 4]);
    mx[e] = smax(smax(mx[e], s[0][e + 8]), s[0][e + 12]);
#pragma unroll
    for (int kb = 1; kb < NK; ++kb) {
      mx[e] = smax(smax(mx[e], s[kb][e]), s[kb][e + 4]);
      mx[e] = smax(smax(mx[e], s[kb][e + 8]), s[kb][e + 12]);
    }
  }
  const float h = smax(smax(smax(mx[0], mx[1]), mx[2]), mx[3]);
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(h), __float_as_uint(h), false, false);
  return smax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// max / sum of a value over lanes l and l ^ 32.
__device__ __forceinline__ float max_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// LDS tile of rows of D 16-bit values (D/8 16-byte chunks per row).  Chunk c of row r lives at
// chunk c ^ swz(r): for D = 128 the low two row bits move to the high two chunk bits, so 16
// consecutive rows at one chunk, or 4 consecutive rows x 4 consecutive chunks, hit 16 distinct
// chunk positions (the two read patterns of the kernels).
template <int D>
__device__ __forceinline__ int swz(int row) {
  if constexpr (D == 128) {
    return ((row & 3) << 2) | ((row >> 2) & 3);
  } else {
    return row & 7;
  }
}

// Index (in 16-byte chunks) of logical chunk c of row r.
template <int D>
__device__ __forceinline__ int chunk_index(int row, int c) {
  return row * (D / 8) + (c ^ swz<D>(row));
}

// Index (in 16-bit elements) of element col of row r (col % 4 == 0 for transpose reads).
template <int D>
__device__ __forceinline__ int elem_index(int row, int col) {
  return row * D + (((col >> 3) ^ swz<D>(row)) << 3) + (col & 7);
}

// Raw buffer resource over `bytes` bytes at `base` (gfx9 data-format word).  Loads at offsets
// at or past `bytes` return zeros, which is how the kernels read ragged tails without branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
  return uint4{v[0], v[1], v[2], v[3]};
}

// Direct load into LDS: each lane fetches 16 bytes at byte offset `off` of the buffer, and lane l's
// bytes land at dst + 16 l (dst must be the same on every lane of the wave).  Loads past the
// buffer's end deliver zeros.  Completion is tracked by the vector-memory counter.  (A device-only
// function: the host pass never sees the cast to the LDS address space.)
__device__ __forceinline__ void buffer_load16_lds(__amdgpu_buffer_rsrc_t r, short* dst, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16, (int)off, 0, 0, 0);
}
// The same with a uniform byte offset `soff` (a scalar register) added to the lane's `off`, so
// that loads whose lane offsets differ by a uniform amount share one address register.
__device__ __forceinline__ void buffer_load16_lds(__amdgpu_buffer_rsrc_t r, short* dst, uint32_t off, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16, (int)off, (int)soff, 0,
                                           0);
}

// Wait for every outstanding memory operation.  Issued once after the loads of loop-invariant
// operands: without it the counter-based waits the compiler places inside the loop (it cannot
// tell that those loads finished in an earlier iteration) also wait for the loop's own
// prefetches, because the counters drain in order, which exposes the full load latency on
// every iteration.
__device__ __forceinline__ void wait_all_loads() { __builtin_amdgcn_s_waitcnt(0); }

// Wait until at most n of this wave's vector-memory operations are outstanding (they complete
// in order, so every older one has finished), without waiting for LDS or scalar loads.
template <int n>
__device__ __forceinline__ void wait_vmem() {
  static_assert(n >= 0 && n < 16, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(0x0F70 | n);   // vmcnt n, expcnt 7, lgkmcnt 15: no other wait
}

// Workgroup barrier after this wave's LDS accesses have completed (s_waitcnt lgkmcnt(0);
// s_barrier): makes LDS writes visible to the other waves without waiting for the direct
// loads in flight, which a full __syncthreads() fence would also wait for.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);   // vmcnt 63, expcnt 7: no wait; lgkmcnt 0
  __builtin_amdgcn_s_barrier();
}

__device__ __forceinline__ i16x4_t ds_read_tr16(const short* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)p);
}

// Transposed A operand from a row-major LDS tile (rows x D, swizzled by swz).  For the 16 rows
// R0 .. R0 + 15 at `base` (R0 a multiple of 16) and columns 32db .. 32db + 31, lane l receives
// A[row = l % 32][k = 8g + e] = tile[R0 + 8(e/4) + 4g + e%4][32db + l % 32]: the rows in the
// order in which a C tile's register r = 8t + e holds them, so the B operand can be a C tile of
// another MFMA packed to 16 bits.  off[hh] = tr_off(lane, db, hh): lane l of each group of 16
// points at row 4(G16/2) + (l%16)/4 + 8hh, columns 32db + 16(G16%2) + 4(l%4) .. + 3.
template <int D>
__device__ __forceinline__ int tr_off(int lane, int db, int hh) {
  const int G16 = lane >> 4, li = lane & 15;
  return elem_index<D>(4 * (G16 >> 1) + (li >> 2) + 8 * hh, 32 * db + 16 * (G16 & 1) + 4 * (li & 3));
}
__device__ __forceinline__ i16x8_t read_tr8(const short* base, const int (&off)[2]) {
  const i16x4_t lo = ds_read_tr16(base + off[0]);
  const i16x4_t hi = ds_read_tr16(base + off[1]);
  return i16x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

}  // namespace eao
