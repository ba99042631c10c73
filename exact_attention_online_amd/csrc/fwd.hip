// Forward pass of exact attention on gfx950: tiled online softmax, fp16/bf16 MFMA.
//
// Method ("FlashAttention (NeurIPS 2022)" notes, "Online Softmax" and "FlashAttention"; the
// FlashAttention-2 OpenReview discussion, author responses): for each block of query rows, walk
// the key/value blocks once, keep a running row maximum m and running denominator l, rescale
// the unnormalised output accumulator by exp(m_old - m_new) when the maximum grows, divide by l
// once at the end, and save the logsumexp.  Causal: key blocks after the last query row of the
// workgroup are skipped and only blocks crossing the diagonal are masked.
//
// gfx950 mapping
//   * grid: one workgroup per (batch, query head, block of BR = 4 * QB * 32 query rows);
//     the 4 waves each own QB * 32 query rows.  Causal launches visit the longest query blocks
//     first (block ids count down), so short blocks fill the tail of the schedule.
//   * transposed formulation: each wave computes S^T = K Q^T and O^T = V^T P^T with
//     v_mfma_f32_32x32x16.  In the S^T accumulator a lane owns one query (column l % 32) and 16
//     keys, so the row maximum and row sum are lane-local; one v_permlane32_swap combines the
//     two lane halves.  O^T's accumulator has the same lane -> query ownership, so the rescale
//     by exp(m_old - m_new) is one multiply per register, and the S^T accumulator, converted
//     to 16-bit, is directly the B operand (P^T) of the second MFMA (k relabelled, see
//     common.hpp).
//   * Q stays in registers for the whole key loop (B operand of S^T).  K and V tiles of BC keys
//     are loaded with 16-byte coalesced global loads into registers one tile ahead and stored
//     into double-buffered, row-padded LDS tiles; K is read with ds_read_b128 and V through
//     ds_read_b64_tr_b16, which delivers V^T fragments without a separate transpose.
//   * softmax in base 2: the running maximum is kept in units of s * scale * log2(e), so each
//     probability is one fma plus one v_exp_f32.
#include <type_traits>

#include "common.hpp"

namespace eao {

// Headroom (log2 units) of the deferred rescaling: probabilities stay <= 2^kStaleMax.
constexpr float kStaleMax = 8.0f;

// LDS tiles use padded rows so that every address is a lane-dependent base plus a constant
// (folded into the instruction's offset field):
//   K tile: row stride D*2 + 16 bytes -- 16 consecutive rows read at one column (ds_read_b128)
//           fall on 16 different 16-byte bank groups;
//   V tile: row stride D*2 + 64 bytes -- 4 consecutive rows x 64 bytes (one 32-lane half of a
//           ds_read_b64_tr_b16) fall on 4 different 64-byte bank groups.
template <int D, int BC>
struct FwdTile {
  static constexpr int CH = D / 8;                 // 16-byte chunks per row
  static constexpr int NLD = BC * CH / 256;        // chunks per thread per tile (K or V)
  static constexpr int KSTR = D + 8;               // K row stride in 16-bit elements
  static constexpr int VSTR = D + 32;              // V row stride in 16-bit elements
  static constexpr int KELEMS = BC * KSTR;
  static constexpr int VELEMS = BC * VSTR;
  static constexpr int BUF = KELEMS + VELEMS;      // 16-bit elements per buffer (K then V)
  static constexpr size_t BYTES = (size_t)2 * BUF * 2;
};

template <bool BF16, int D, int QB, int BC, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void attn_fwd_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    uint16_t* __restrict__ O, float* __restrict__ LSE, int Hq, int Hkv, int N, int BH, int nqb,
    float c /* softmax_scale * log2(e) */) {
  using T = FwdTile<D, BC>;
  constexpr int CH = T::CH, NLD = T::NLD, KK = D / 16, DB = D / 32, KB = BC / 32;
  constexpr int BR = 4 * QB * 32;
  constexpr int KSTR = T::KSTR, VSTR = T::VSTR;
  extern __shared__ uint4 smem[];   // [2 buffers][K tile, V tile]
  short* const sm = (short*)smem;
  auto Ks = [&](int buf) { return sm + buf * T::BUF; };
  auto Vs = [&](int buf) { return sm + buf * T::BUF + T::KELEMS; };

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, g = lane >> 5, l32 = lane & 31;
  const int L = blockIdx.x;
  const int qblk = CAUSAL ? (nqb - 1 - L / BH) : (L / BH);
  const int bh = L % BH;
  const int h = bh % Hq, b = bh / Hq;
  const int kvh = h / (Hq / Hkv);
  const size_t q_off = ((size_t)b * Hq + h) * (size_t)N * D;
  const size_t kv_off = ((size_t)b * Hkv + kvh) * (size_t)N * D;
  const uint16_t* Qp = Q + q_off;
  const uint16_t* Kp = K + kv_off;
  const uint16_t* Vp = V + kv_off;

  const int q0 = qblk * BR;
  const int qw = q0 + w * QB * 32;          // first query row of this wave
  const int qw_last = qw + QB * 32 - 1;

  // Q^T fragments (B operand): lane holds Q[row][16kk + 8g .. +7]
  i16x8_t qf[QB][KK];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = qw + 32 * qb + l32;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      if (row < N) {
        qf[qb][kk] = __builtin_bit_cast(i16x8_t, *(const uint4*)(Qp + (size_t)row * D + 16 * kk + 8 * g));
      } else {
        qf[qb][kk] = i16x8_t{0, 0, 0, 0, 0, 0, 0, 0};
      }
    }
  }

  wait_all_loads();

  f32x16_t o[QB][DB];
  float m[QB], l[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m[qb] = -INFINITY;
    l[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) o[qb][db] = f32x16_t{};
  }

  const int kend = CAUSAL ? min(N, q0 + BR) : N;
  const int ntiles = (kend + BC - 1) / BC;

  // K/V of this head through bounds-checked buffer loads: keys >= N read as zeros
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(Kp, (uint32_t)N * D * 2);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(Vp, (uint32_t)N * D * 2);
  uint4 kreg[NLD], vreg[NLD];
  auto load_tile = [&](int kt0) {
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int cidx = tid + 256 * i;
      const int row = cidx / CH, ch = cidx % CH;
      const uint32_t off = ((uint32_t)(kt0 + row) * D + ch * 8) * 2;
      kreg[i] = buffer_load16(krs, off);
      vreg[i] = buffer_load16(vrs, off);
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int cidx = tid + 256 * i;
      const int row = cidx / CH, ch = cidx % CH;
      *(uint4*)(Ks(buf) + row * KSTR + ch * 8) = kreg[i];
      *(uint4*)(Vs(buf) + row * VSTR + ch * 8) = vreg[i];
    }
  };

  // One key tile: S^T, (masked) online softmax, O^T += V^T P^T.  MASK selects the variant with
  // causal / key-tail masking; only tiles that cross the diagonal or the end of the keys need it.
  auto tile = [&](int j, auto mask_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const int kt0 = j * BC;
    const bool has_next = j + 1 < ntiles;
    if (has_next) load_tile(kt0 + BC);

    const bool active = (qw < N) && (!CAUSAL || kt0 <= qw_last);
    if (active) {
      const short* Kb = Ks(j & 1);
      const short* Vb = Vs(j & 1);
      // ---- S^T = K Q^T
      f32x16_t s[QB][KB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) s[qb][kb] = f32x16_t{};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          const i16x8_t a = __builtin_bit_cast(i16x8_t, *(const uint4*)(Kb + (32 * kb + l32) * KSTR + 16 * kk + 8 * g));
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) s[qb][kb] = mfma32x32x16<BF16>(a, qf[qb][kk], s[qb][kb]);
        }
      }
      // ---- online softmax
      i16x8_t pf[QB][KB][2];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        if constexpr (MASK) {
          const int qrow = qw + 32 * qb + l32;
#pragma unroll
          for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = kt0 + 32 * kb + 8 * (r >> 2) + 4 * g + (r & 3);
              if (key >= N || (CAUSAL && key > qrow)) s[qb][kb][r] = -INFINITY;
            }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[qb][kb][r]);
        const float mt = max_halves(mx) * c;
        // The accumulator is rescaled only when some row's maximum has grown by more than
        // kStaleMax (log2 units) since the last rescale; otherwise the stale maximum is kept,
        // probabilities stay <= 2^kStaleMax, and the final division by l (computed against the
        // same maximum) gives the same result.
        // The decision is per row (alpha is exactly 1 where the row keeps its maximum), so a
        // row's result never depends on other rows; the branch only skips the multiplies when
        // no row of the wave needs them.
        const bool grow = mt > m[qb] + kStaleMax;
        if (__builtin_amdgcn_ballot_w64(grow) != 0) {
          float alpha = grow ? __builtin_amdgcn_exp2f(m[qb] - mt) : 1.f;
          // an opaque (volatile) definition of alpha pins the multiplies below inside this
          // branch; left alone, the compiler hoists them and runs them on every tile
          asm volatile("" : "+v"(alpha));
          m[qb] = grow ? mt : m[qb];
          l[qb] *= alpha;
#pragma unroll
          for (int db = 0; db < DB; ++db) o[qb][db] *= alpha;
        }
        const float muse = (m[qb] == -INFINITY) ? 0.f : m[qb];
        float rs = 0.f;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float p = __builtin_amdgcn_exp2f(s[qb][kb][r] * c - muse);
            s[qb][kb][r] = p;
            rs += p;
          }
        l[qb] += rs;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          pf[qb][kb][0] = pack8<BF16>(s[qb][kb], 0);
          pf[qb][kb][1] = pack8<BF16>(s[qb][kb], 8);
        }
      }
      // ---- O^T += V^T P^T
      const int G16 = lane >> 4, li = lane & 15;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int krow = 32 * kb + 16 * t + 4 * (G16 >> 1) + (li >> 2);
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const int col = 32 * db + 16 * (G16 & 1) + 4 * (li & 3);
            const i16x4_t lo = ds_read_tr16(Vb + krow * VSTR + col);
            const i16x4_t hi = ds_read_tr16(Vb + (krow + 8) * VSTR + col);
            const i16x8_t a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) o[qb][db] = mfma32x32x16<BF16>(a, pf[qb][kb][t], o[qb][db]);
          }
        }
    }

    if (has_next) store_tile((j + 1) & 1);
    __syncthreads();
  };

  load_tile(0);
  store_tile(0);
  __syncthreads();

  // tiles [0, jmask) need no masking for any wave of the workgroup
  const int jmask = min(ntiles, CAUSAL ? min(q0, N) / BC : N / BC);
  int j = 0;
  for (; j < jmask; ++j) tile(j, std::false_type{});
  for (; j < ntiles; ++j) tile(j, std::true_type{});

  // ---- epilogue: O = O_acc / l, LSE = ln2 * (m + log2 l)
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float lt = sum_halves(l[qb]);
    const float inv = 1.f / lt;
    const int qrow = qw + 32 * qb + l32;
    if (qrow < N) {
      uint16_t* Op = O + q_off + (size_t)qrow * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int d0 = 32 * db + 8 * rr + 4 * g;
          uint2 pk;
          pk.x = pack2<BF16>(o[qb][db][4 * rr + 0] * inv, o[qb][db][4 * rr + 1] * inv);
          pk.y = pack2<BF16>(o[qb][db][4 * rr + 2] * inv, o[qb][db][4 * rr + 3] * inv);
          *(uint2*)(Op + d0) = pk;
        }
      if (g == 0) LSE[(size_t)bh * N + qrow] = (m[qb] + __log2f(lt)) * kLn2;
    }
  }
}

template <bool BF16, int D, int QB, int BC, bool CAUSAL>
static hipError_t launch_fwd_t(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
                               int Hkv, int N, float scale, hipStream_t stream) {
  constexpr int BR = 4 * QB * 32;
  const int nqb = (N + BR - 1) / BR;
  const int BH = B * Hq;
  const size_t lds = FwdTile<D, BC>::BYTES;
  auto kern = attn_fwd_kernel<BF16, D, QB, BC, CAUSAL>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(nqb * BH), dim3(256), lds, stream, (const uint16_t*)q, (const uint16_t*)k,
                     (const uint16_t*)v, (uint16_t*)o, lse, Hq, Hkv, N, BH, nqb, scale * kLog2e);
  return hipGetLastError();
}

hipError_t launch_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv,
                      int N, int d, bool causal, float scale, bool bf16, hipStream_t stream) {
#define EAO_FWD(BF, DD, CA) \
  return launch_fwd_t<BF, DD, 1, 64, CA>(q, k, v, o, lse, B, Hq, Hkv, N, scale, stream)
  if (bf16) {
    if (d == 128) { if (causal) EAO_FWD(true, 128, true); else EAO_FWD(true, 128, false); }
    else { if (causal) EAO_FWD(true, 64, true); else EAO_FWD(true, 64, false); }
  } else {
    if (d == 128) { if (causal) EAO_FWD(false, 128, true); else EAO_FWD(false, 128, false); }
    else { if (causal) EAO_FWD(false, 64, true); else EAO_FWD(false, 64, false); }
  }
#undef EAO_FWD
}

}  // namespace eao
