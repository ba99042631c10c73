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
//     into a double-buffered, XOR-swizzled LDS tile; K is read with ds_read_b128 and V through
//     ds_read_b64_tr_b16, which delivers V^T fragments without a separate transpose.
//   * softmax in base 2: the running maximum is kept in units of s * scale * log2(e), so each
//     probability is one fma plus one v_exp_f32.
#include "common.hpp"

namespace eao {

template <int D, int BC>
struct FwdTile {
  static constexpr int CH = D / 8;                 // 16-byte chunks per row
  static constexpr int NLD = BC * CH / 256;        // chunks per thread per tile (K or V)
  static constexpr int ELEMS = BC * D;             // 16-bit elements per tile
};

template <bool BF16, int D, int QB, int BC, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void attn_fwd_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    uint16_t* __restrict__ O, float* __restrict__ LSE, int Hq, int Hkv, int N, int BH, int nqb,
    float c /* softmax_scale * log2(e) */) {
  using T = FwdTile<D, BC>;
  constexpr int CH = T::CH, NLD = T::NLD, KK = D / 16, DB = D / 32, KB = BC / 32;
  constexpr int BR = 4 * QB * 32;
  extern __shared__ uint4 smem[];   // [2 buffers][K tile, V tile]
  auto Ks = [&](int buf) { return smem + buf * 2 * BC * CH; };
  auto Vs = [&](int buf) { return smem + buf * 2 * BC * CH + BC * CH; };

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

  uint4 kreg[NLD], vreg[NLD];
  auto load_tile = [&](int kt0) {
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int cidx = tid + 256 * i;
      const int row = cidx / CH, ch = cidx % CH;
      const int key = kt0 + row;
      if (key < N) {
        kreg[i] = *(const uint4*)(Kp + (size_t)key * D + ch * 8);
        vreg[i] = *(const uint4*)(Vp + (size_t)key * D + ch * 8);
      } else {
        kreg[i] = uint4{0, 0, 0, 0};
        vreg[i] = uint4{0, 0, 0, 0};
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int cidx = tid + 256 * i;
      const int row = cidx / CH, ch = cidx % CH;
      Ks(buf)[chunk_index<D>(row, ch)] = kreg[i];
      Vs(buf)[chunk_index<D>(row, ch)] = vreg[i];
    }
  };

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int j = 0; j < ntiles; ++j) {
    const int kt0 = j * BC;
    const bool has_next = j + 1 < ntiles;
    if (has_next) load_tile(kt0 + BC);

    const bool active = (qw < N) && (!CAUSAL || kt0 <= qw_last);
    if (active) {
      const uint4* Kb = Ks(j & 1);
      const short* Vb = (const short*)Vs(j & 1);
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
          const i16x8_t a = __builtin_bit_cast(i16x8_t, Kb[chunk_index<D>(32 * kb + l32, 2 * kk + g)]);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) s[qb][kb] = mfma32x32x16<BF16>(a, qf[qb][kk], s[qb][kb]);
        }
      }
      // ---- mask, online softmax
      const bool need_mask = (kt0 + BC > N) || (CAUSAL && kt0 + BC - 1 > qw);
      i16x8_t pf[QB][KB][2];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const int qrow = qw + 32 * qb + l32;
        if (need_mask) {
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
        mx = max_halves(mx);
        const float mnew = fmaxf(m[qb], mx * c);
        const float muse = (mnew == -INFINITY) ? 0.f : mnew;
        const float alpha = __builtin_amdgcn_exp2f(m[qb] - muse);
        m[qb] = mnew;
        float rs = 0.f;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float p = __builtin_amdgcn_exp2f(s[qb][kb][r] * c - muse);
            s[qb][kb][r] = p;
            rs += p;
          }
        l[qb] = l[qb] * alpha + rs;
#pragma unroll
        for (int db = 0; db < DB; ++db) o[qb][db] *= alpha;
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
            const i16x4_t lo = ds_read_tr16(Vb + elem_index<D>(krow, col));
            const i16x4_t hi = ds_read_tr16(Vb + elem_index<D>(krow + 8, col));
            const i16x8_t a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) o[qb][db] = mfma32x32x16<BF16>(a, pf[qb][kb][t], o[qb][db]);
          }
        }
    }

    if (has_next) store_tile((j + 1) & 1);
    __syncthreads();
  }

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
  const size_t lds = (size_t)4 * BC * D * 2;
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
