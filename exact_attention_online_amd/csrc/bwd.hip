// Backward pass of exact attention on gfx950 (fp16/bf16 MFMA, fp32 accumulation).
//
// Method ("FlashAttention (NeurIPS 2022)" notes, "Backward - Recomputation"; FlashAttention-2
// OpenReview discussion: dV = P^T dO, the logsumexp saved by the forward, the backward's
// sharing of the query-gradient update, grouped-query attention): nothing of size N x N is
// stored; S and P are recomputed block by block from Q, K and the saved LSE, and
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D) with D_i = rowsum(dO_i * O_i),
//   dK = scale dS^T Q,  dQ = scale dS K.
//
// Three kernels on the caller's stream:
//   1. bwd_pre: D = rowsum(dO * O) (fp32) and a zeroed fp32 dQ accumulator (workspace).
//   2. bwd_main: one workgroup per (batch, K/V head, block of 128 keys).  Each of the 4 waves
//      owns 32 keys and keeps K and V fragments, and its dK^T and dV^T accumulators, in
//      registers for the whole kernel.  The workgroup walks every query head of the K/V head's
//      group and every query block of 64 rows (causal: from the diagonal on), so dK and dV are
//      summed over the group without atomics.  Q and dO tiles (plus LSE and D) are prefetched
//      into registers one block ahead and stored into double-buffered swizzled LDS.  Per block:
//        S = Q K^T and dP = dO V^T    (A = Q / dO rows via ds_read_b128, B = K / V registers;
//                                      in the accumulator a lane owns one key column)
//        P = exp2(S * scale * log2e - LSE * log2e), masked;  dS = P * (dP - D)
//        dV^T += dO^T P, dK^T += Q^T dS (A = dO^T / Q^T via ds_read_b64_tr_b16, B = P / dS
//                                      straight from the accumulator registers)
//        dS^T goes to LDS (double buffered); after one barrier every wave computes
//        dQ[64 rows, its 32-column slice] = dS K over all 128 keys (A = dS via transpose reads,
//        B = K fragments held in registers) and adds it into the fp32 accumulator with
//        global atomics.
//   3. bwd_dq_convert: dQ = scale * accumulator, rounded to the input dtype.
#include "common.hpp"

namespace eao {

constexpr int kBwdKeys = 128;   // keys per workgroup (32 per wave)
constexpr int kBwdRows = 64;    // query rows per step

size_t bwd_workspace_bytes(int B, int Hq, int N, int d) {
  const size_t rows = (size_t)B * Hq * N;
  return ((rows * 4 + 255) / 256) * 256 + rows * (size_t)d * 4;
}

// ------------------------------------------------------------------ 1. preprocess
// 16 lanes per row; each lane handles 8 of the row's d elements.
template <bool BF16, int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const uint16_t* __restrict__ O, const uint16_t* __restrict__ dO,
                                                      float* __restrict__ Dsum, float* __restrict__ dq_acc,
                                                      size_t rows) {
  constexpr int LPR = 16;                 // lanes per row
  constexpr int EPL = D / LPR;            // elements per lane (8 for d = 128, 4 for d = 64)
  const size_t row = (size_t)blockIdx.x * (256 / LPR) + threadIdx.x / LPR;
  const int sub = threadIdx.x % LPR;
  float acc = 0.f;
  if (row < rows) {
    const uint16_t* op = O + row * D + sub * EPL;
    const uint16_t* dp = dO + row * D + sub * EPL;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc += to_float<BF16>(op[e]) * to_float<BF16>(dp[e]);
    float4* z = (float4*)(dq_acc + row * D + sub * EPL);
#pragma unroll
    for (int e = 0; e < EPL / 4; ++e) z[e] = float4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, LPR);
  if (row < rows && sub == 0) Dsum[row] = acc;
}

// ------------------------------------------------------------------ 3. dQ convert
template <bool BF16>
__global__ __launch_bounds__(256) void bwd_dq_convert_kernel(const float* __restrict__ acc, uint16_t* __restrict__ dq,
                                                             size_t n4, float scale) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  const float4 a = ((const float4*)acc)[i];
  uint2 pk;
  pk.x = pack2<BF16>(a.x * scale, a.y * scale);
  pk.y = pack2<BF16>(a.z * scale, a.w * scale);
  ((uint2*)dq)[i] = pk;
}

// ------------------------------------------------------------------ 2. main
template <int D>
struct BwdSmem {
  static constexpr int TILE = kBwdRows * D;                 // 16-bit elements of a Q or dO tile
  static constexpr int DST = kBwdKeys * kBwdRows;           // 16-bit elements of the dS^T tile
  static constexpr int KT = kBwdKeys * D;                   // 16-bit elements of the K tile
  // layout (16-bit units): [buf0: Q, dO][buf1: Q, dO][dS^T x2][K], then floats [buf][LSE2, D] x 64
  static constexpr int Q_OFF(int buf) { return buf * 2 * TILE; }
  static constexpr int DO_OFF(int buf) { return buf * 2 * TILE + TILE; }
  static constexpr int DS_OFF(int buf) { return 4 * TILE + buf * DST; }
  static constexpr int K_OFF = 4 * TILE + 2 * DST;
  static constexpr int F_OFF = K_OFF + KT;                  // start of the float area (16-bit units)
  static constexpr size_t BYTES = (size_t)F_OFF * 2 + 2 * 2 * kBwdRows * 4;
};

template <bool BF16, int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void bwd_main_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Dsum,
    float* __restrict__ dq_acc, uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, int Hq, int Hkv, int N,
    int nkb, float c /* scale * log2(e) */, float scale) {
  using SM = BwdSmem<D>;
  constexpr int CH = D / 8, KK = D / 16, DB = D / 32;
  constexpr int NLD = kBwdRows * CH / 256;          // 16-byte chunks per thread per tile
  constexpr int DQP = D / 64;                       // (row half, 32-column slice) pairs per wave in dQ
  extern __shared__ uint4 smem_u4[];
  short* sm = (short*)smem_u4;
  float* smf = (float*)(sm + SM::F_OFF);            // [buf][0: LSE2 | 1: D][64]

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, g = lane >> 5, l32 = lane & 31;
  const int G16 = lane >> 4, li = lane & 15;
  const int G = Hq / Hkv;
  // key block major: under causal masking the first key blocks see the most query rows, so
  // the heaviest workgroups of every head start first
  const int L = blockIdx.x;
  const int BHkv = gridDim.x / nkb;
  const int kblk = L / BHkv;
  const int bkv = L % BHkv;
  const int b = bkv / Hkv, kvh = bkv % Hkv;
  const int k0 = kblk * kBwdKeys;
  const int kw = k0 + 32 * w;                       // this wave's first key
  const size_t kv_off = ((size_t)b * Hkv + kvh) * (size_t)N * D;

  // ---- persistent fragments: K, V rows of this wave (B operands of S and dP)
  i16x8_t kf[KK], vf[KK];
  {
    const int key = kw + l32;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      if (key < N) {
        kf[kk] = __builtin_bit_cast(i16x8_t, *(const uint4*)(K + kv_off + (size_t)key * D + 16 * kk + 8 * g));
        vf[kk] = __builtin_bit_cast(i16x8_t, *(const uint4*)(V + kv_off + (size_t)key * D + 16 * kk + 8 * g));
      } else {
        kf[kk] = i16x8_t{0, 0, 0, 0, 0, 0, 0, 0};
        vf[kk] = i16x8_t{0, 0, 0, 0, 0, 0, 0, 0};
      }
    }
  }
  // ---- the workgroup's K tile in LDS (B operand of dQ = dS K, read transposed)
  {
    uint4* kt = (uint4*)(sm + SM::K_OFF);
#pragma unroll
    for (int i = 0; i < kBwdKeys * CH / 256; ++i) {
      const int cidx = tid + 256 * i;
      const int row = cidx / CH, ch = cidx % CH;
      const int key = k0 + row;
      kt[chunk_index<D>(row, ch)] =
          key < N ? *(const uint4*)(K + kv_off + (size_t)key * D + ch * 8) : uint4{0, 0, 0, 0};
    }
  }

  f32x16_t dvacc[DB], dkacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    dvacc[db] = f32x16_t{};
    dkacc[db] = f32x16_t{};
  }

  const int nqb = (N + kBwdRows - 1) / kBwdRows;
  const int qstart = CAUSAL ? (k0 / kBwdRows) : 0;
  const int per_head = nqb - qstart;
  const int total = G * per_head;

  uint4 qreg[NLD], doreg[NLD];
  float lse_reg = 0.f, d_reg = 0.f;
  auto load_tile = [&](int it) {
    const int hh = it / per_head;
    const int q0 = (qstart + it % per_head) * kBwdRows;
    const size_t q_off = ((size_t)b * Hq + (size_t)kvh * G + hh) * (size_t)N;
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int cidx = tid + 256 * i;
      const int row = cidx / CH, ch = cidx % CH;
      const int q = q0 + row;
      if (q < N) {
        qreg[i] = *(const uint4*)(Q + (q_off + q) * D + ch * 8);
        doreg[i] = *(const uint4*)(dO + (q_off + q) * D + ch * 8);
      } else {
        qreg[i] = uint4{0, 0, 0, 0};
        doreg[i] = uint4{0, 0, 0, 0};
      }
    }
    if (tid < kBwdRows) {
      const int q = q0 + tid;
      // rows past the end get LSE = +inf, so their probabilities are exactly 0
      lse_reg = q < N ? LSE[q_off + q] * kLog2e : INFINITY;
      d_reg = q < N ? Dsum[q_off + q] : 0.f;
    }
  };
  auto store_tile = [&](int buf) {
    uint4* qs = (uint4*)(sm + SM::Q_OFF(buf));
    uint4* ds = (uint4*)(sm + SM::DO_OFF(buf));
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int cidx = tid + 256 * i;
      const int row = cidx / CH, ch = cidx % CH;
      qs[chunk_index<D>(row, ch)] = qreg[i];
      ds[chunk_index<D>(row, ch)] = doreg[i];
    }
    if (tid < kBwdRows) {
      smf[buf * 2 * kBwdRows + tid] = lse_reg;
      smf[buf * 2 * kBwdRows + kBwdRows + tid] = d_reg;
    }
  };

  if (total > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  for (int it = 0; it < total; ++it) {
    const int buf = it & 1;
    const bool has_next = it + 1 < total;
    if (has_next) load_tile(it + 1);
    const int hh = it / per_head;
    const int h = kvh * G + hh;
    const int q0 = (qstart + it % per_head) * kBwdRows;
    const short* Qs = sm + SM::Q_OFF(buf);
    const short* dOs = sm + SM::DO_OFF(buf);
    short* dSs = sm + SM::DS_OFF(buf);
    const float* lse_s = smf + buf * 2 * kBwdRows;
    const float* d_s = lse_s + kBwdRows;

    const bool active = !(CAUSAL && q0 + kBwdRows - 1 < kw) && kw < N;
    if (active) {
      const int key = kw + l32;
      const bool need_mask = (CAUSAL && q0 < kw + 31) || (k0 + kBwdKeys > N);
      const int krow_ds = 32 * w + l32;
#pragma unroll
      for (int qs = 0; qs < 2; ++qs) {
        // S = Q K^T, dP = dO V^T for rows 32qs .. 32qs+31 of the block
        f32x16_t s = f32x16_t{}, dp = f32x16_t{};
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          const int ci = chunk_index<D>(32 * qs + l32, 2 * kk + g);
          const i16x8_t aq = __builtin_bit_cast(i16x8_t, ((const uint4*)Qs)[ci]);
          const i16x8_t ado = __builtin_bit_cast(i16x8_t, ((const uint4*)dOs)[ci]);
          s = mfma32x32x16<BF16>(aq, kf[kk], s);
          dp = mfma32x32x16<BF16>(ado, vf[kk], dp);
        }
        // P and dS; lane owns key kw + l32, register r holds query q0 + 32qs + 8(r/4) + 4g + r%4
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int qr = 32 * qs + 8 * rr + 4 * g;
          const float4 l4 = *(const float4*)(lse_s + qr);
          const float4 d4 = *(const float4*)(d_s + qr);
          const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
          const float dv4[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * rr + e;
            float p = __builtin_amdgcn_exp2f(s[r] * c - lv[e]);
            if (need_mask) {
              const int q = q0 + qr + e;
              if (key >= N || (CAUSAL && key > q)) p = 0.f;
            }
            s[r] = p;
            dp[r] = p * (dp[r] - dv4[e]);
          }
        }
        const i16x8_t pb[2] = {pack8<BF16>(s, 0), pack8<BF16>(s, 8)};
        const i16x8_t sb[2] = {pack8<BF16>(dp, 0), pack8<BF16>(dp, 8)};
        // dV^T += dO^T P ; dK^T += Q^T dS   (k = query rows, slot (g, e) as in the forward)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int qrow = 32 * qs + 16 * t + 4 * (G16 >> 1) + (li >> 2);
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const int col = 32 * db + 16 * (G16 & 1) + 4 * (li & 3);
            const i16x4_t a0 = ds_read_tr16(dOs + elem_index<D>(qrow, col));
            const i16x4_t a1 = ds_read_tr16(dOs + elem_index<D>(qrow + 8, col));
            const i16x8_t ado = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
            dvacc[db] = mfma32x32x16<BF16>(ado, pb[t], dvacc[db]);
            const i16x4_t b0 = ds_read_tr16(Qs + elem_index<D>(qrow, col));
            const i16x4_t b1 = ds_read_tr16(Qs + elem_index<D>(qrow + 8, col));
            const i16x8_t aq = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
            dkacc[db] = mfma32x32x16<BF16>(aq, sb[t], dkacc[db]);
          }
        }
        // dS^T -> LDS: row = local key, 4 consecutive query columns per 8-byte store
        // (sb holds the same bf16 values: slot (g, e) of half t is query 16t + 8(e/4) + 4g + e%4)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
          const u32x4_t wv = __builtin_bit_cast(u32x4_t, sb[t]);
          *(uint2*)(dSs + elem_index<kBwdRows>(krow_ds, 32 * qs + 16 * t + 4 * g)) = uint2{wv[0], wv[1]};
          *(uint2*)(dSs + elem_index<kBwdRows>(krow_ds, 32 * qs + 16 * t + 8 + 4 * g)) = uint2{wv[2], wv[3]};
        }
      }
    } else {
      const int krow = 32 * w + l32;
#pragma unroll
      for (int cc = 0; cc < kBwdRows / 4; cc += 2) {
        *(uint2*)(dSs + elem_index<kBwdRows>(krow, 4 * (cc + g))) = uint2{0, 0};
      }
    }

    if (has_next) store_tile(buf ^ 1);
    __syncthreads();

    // ---- dQ[q0 + 64 rows][column slice] += dS K over the workgroup's 128 keys
    const size_t q_off = ((size_t)b * Hq + h) * (size_t)N;
#pragma unroll
    for (int j = 0; j < DQP; ++j) {
      const int p = w * DQP + j;
      const int qs = p & 1, dsl = p >> 1;
      f32x16_t acc = f32x16_t{};
      const int colq = 32 * qs + 16 * (G16 & 1) + 4 * (li & 3);
      const int cold = 32 * dsl + 16 * (G16 & 1) + 4 * (li & 3);
      const short* Kt = sm + SM::K_OFF;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        // slot (g, e) <-> key 16t + 8g + e on both operands
        const int krow = 16 * t + 8 * (G16 >> 1) + (li >> 2);
        const i16x4_t a0 = ds_read_tr16(dSs + elem_index<kBwdRows>(krow, colq));
        const i16x4_t a1 = ds_read_tr16(dSs + elem_index<kBwdRows>(krow + 4, colq));
        const i16x8_t a = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
        const i16x4_t b0 = ds_read_tr16(Kt + elem_index<D>(krow, cold));
        const i16x4_t b1 = ds_read_tr16(Kt + elem_index<D>(krow + 4, cold));
        const i16x8_t bk = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
        acc = mfma32x32x16<BF16>(a, bk, acc);
      }
      // acc: C[row = query 8(r/4) + 4g + r%4][col = d within slice] ... transposed roles:
      // A rows are queries (dS), B columns are d (K) -> C[query][d]
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int q = q0 + 32 * qs + 8 * (r >> 2) + 4 * g + (r & 3);
        if (q < N) atomicAdd(dq_acc + (q_off + q) * D + 32 * dsl + l32, acc[r]);
      }
    }
  }

  // ---- epilogue: dV, dK (lane owns key kw + l32; register r holds d = 32db + 8(r/4) + 4g + r%4)
  const int key = kw + l32;
  if (key < N) {
    uint16_t* dvp = dV + kv_off + (size_t)key * D;
    uint16_t* dkp = dK + kv_off + (size_t)key * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int d0 = 32 * db + 8 * rr + 4 * g;
        uint2 pv, pk;
        pv.x = pack2<BF16>(dvacc[db][4 * rr + 0], dvacc[db][4 * rr + 1]);
        pv.y = pack2<BF16>(dvacc[db][4 * rr + 2], dvacc[db][4 * rr + 3]);
        pk.x = pack2<BF16>(dkacc[db][4 * rr + 0] * scale, dkacc[db][4 * rr + 1] * scale);
        pk.y = pack2<BF16>(dkacc[db][4 * rr + 2] * scale, dkacc[db][4 * rr + 3] * scale);
        *(uint2*)(dvp + d0) = pv;
        *(uint2*)(dkp + d0) = pk;
      }
  }
}

static float* workspace_acc(void* workspace, size_t rows) {
  return (float*)((char*)workspace + ((rows * 4 + 255) / 256) * 256);
}

template <bool BF16, int D>
static hipError_t launch_bwd_pre_t(const void* o, const void* dout, size_t rows, void* workspace,
                                   hipStream_t stream) {
  hipLaunchKernelGGL((bwd_pre_kernel<BF16, D>), dim3((unsigned)((rows + 15) / 16)), dim3(256), 0, stream,
                     (const uint16_t*)o, (const uint16_t*)dout, (float*)workspace, workspace_acc(workspace, rows),
                     rows);
  return hipGetLastError();
}

template <bool BF16, int D, bool CAUSAL>
static hipError_t launch_bwd_main_t(const void* q, const void* k, const void* v, const void* dout, const float* lse,
                                    void* dk, void* dv, int B, int Hq, int Hkv, int N, float scale, void* workspace,
                                    hipStream_t stream) {
  const size_t rows = (size_t)B * Hq * N;
  const int nkb = (N + kBwdKeys - 1) / kBwdKeys;
  auto kern = bwd_main_kernel<BF16, D, CAUSAL>;
  const size_t lds = BwdSmem<D>::BYTES;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(nkb * B * Hkv), dim3(256), lds, stream, (const uint16_t*)q, (const uint16_t*)k,
                     (const uint16_t*)v, (const uint16_t*)dout, lse, (const float*)workspace,
                     workspace_acc(workspace, rows), (uint16_t*)dk, (uint16_t*)dv, Hq, Hkv, N, nkb,
                     scale * kLog2e, scale);
  return hipGetLastError();
}

template <bool BF16>
static hipError_t launch_bwd_convert_t(void* dq, size_t rows, int d, float scale, void* workspace,
                                       hipStream_t stream) {
  const size_t n4 = rows * d / 4;
  hipLaunchKernelGGL((bwd_dq_convert_kernel<BF16>), dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, stream,
                     (const float*)workspace_acc(workspace, rows), (uint16_t*)dq, n4, scale);
  return hipGetLastError();
}

hipError_t launch_bwd_pre(const void* o, const void* dout, int B, int Hq, int N, int d, bool bf16, void* workspace,
                          hipStream_t stream) {
  const size_t rows = (size_t)B * Hq * N;
  if (bf16) return d == 128 ? launch_bwd_pre_t<true, 128>(o, dout, rows, workspace, stream)
                            : launch_bwd_pre_t<true, 64>(o, dout, rows, workspace, stream);
  return d == 128 ? launch_bwd_pre_t<false, 128>(o, dout, rows, workspace, stream)
                  : launch_bwd_pre_t<false, 64>(o, dout, rows, workspace, stream);
}

hipError_t launch_bwd_main(const void* q, const void* k, const void* v, const void* dout, const float* lse, void* dk,
                           void* dv, int B, int Hq, int Hkv, int N, int d, bool causal, float scale, bool bf16,
                           void* workspace, hipStream_t stream) {
#define EAO_BWD(BF, DD, CA) \
  return launch_bwd_main_t<BF, DD, CA>(q, k, v, dout, lse, dk, dv, B, Hq, Hkv, N, scale, workspace, stream)
  if (bf16) {
    if (d == 128) { if (causal) EAO_BWD(true, 128, true); else EAO_BWD(true, 128, false); }
    else { if (causal) EAO_BWD(true, 64, true); else EAO_BWD(true, 64, false); }
  } else {
    if (d == 128) { if (causal) EAO_BWD(false, 128, true); else EAO_BWD(false, 128, false); }
    else { if (causal) EAO_BWD(false, 64, true); else EAO_BWD(false, 64, false); }
  }
#undef EAO_BWD
}

hipError_t launch_bwd_convert(void* dq, int B, int Hq, int N, int d, float scale, bool bf16, void* workspace,
                              hipStream_t stream) {
  const size_t rows = (size_t)B * Hq * N;
  return bf16 ? launch_bwd_convert_t<true>(dq, rows, d, scale, workspace, stream)
              : launch_bwd_convert_t<false>(dq, rows, d, scale, workspace, stream);
}

}  // namespace eao
