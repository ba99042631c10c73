// Backward pass of exact attention on gfx950 (fp16/bf16 MFMA, fp32 accumulation).
//
// Method ("FlashAttention (NeurIPS 2022)" notes, "Backward - Recomputation"; FlashAttention-2
// OpenReview discussion: dV = P^T dO, the logsumexp saved by the forward, grouped-query
// attention): nothing of size N x N is stored; S and P are recomputed block by block from Q, K
// and the saved LSE, and
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D) with D_i = rowsum(dO_i * O_i),
//   dK = scale dS^T Q,  dQ = scale dS K.
//
// Three kernels on the caller's stream, none of them atomic:
//   1. bwd_pre: D = rowsum(dO * O) in fp32 (the workspace).
//   2. bwd_dkdv: one workgroup per (batch, K/V head, block of 128 keys); each of the 4 waves
//      owns 32 keys and keeps their K and V fragments and its dK^T, dV^T accumulators in
//      registers for the whole kernel.  The workgroup walks every query head of the K/V head's
//      group and every block of 64 query rows (causal: from the diagonal on), so dK and dV are
//      summed over the group in registers.  Q and dO tiles (plus LSE and D) are prefetched into
//      registers one block ahead and stored into double-buffered swizzled LDS.  Per block:
//        S = Q K^T, dP = dO V^T   (A = Q / dO rows via ds_read_b128, B = K / V registers; a lane
//                                  owns one key column of the accumulator)
//        P = exp2(S * scale * log2e - LSE * log2e) (causal mask on the diagonal blocks only);
//        dS = P * (dP - D);  dV^T += dO^T P, dK^T += Q^T dS with P and dS taken straight from
//        the accumulators (dO^T, Q^T via ds_read_b64_tr_b16).
//   3. bwd_dq: one workgroup per (batch, query head, block of 128 query rows), shaped like the
//      forward: a lane owns one query row, so LSE and D are one register each.  Per key tile:
//        S^T = K Q^T, dP^T = V dO^T, dS^T = P^T * (dP^T - D), dQ^T += K^T dS^T,
//      with dS^T fed from the accumulator into the last MFMA (k relabelled as in the forward)
//      and K^T read through ds_read_b64_tr_b16; dQ = scale * dQ^T is written once at the end.
// Splitting dQ off costs two extra contractions (S and dP are recomputed) but replaces the
// fp32 atomic accumulation of dQ, whose ordered completion stalled the loads of the
// key-stationary kernel, with plain register accumulation.
//
// Keys or query rows past N read as zeros (bounds-checked buffer loads).  Zero K/V rows and
// zero Q/dO/D rows make every contribution that crosses the end of the sequence vanish exactly,
// so only the causal diagonal is masked.
#include <type_traits>

#include "common.hpp"

namespace eao {

constexpr int kBwdKeys = 128;   // keys per dK/dV workgroup (32 per wave)
constexpr int kBwdRows = 64;    // query rows per dK/dV step
constexpr int kDqRows = 128;    // query rows per dQ workgroup (32 per wave)
constexpr int kDqKeys = 64;     // keys per dQ step

size_t bwd_workspace_bytes(int B, int Hq, int N, int d) {
  (void)d;
  return (((size_t)B * Hq * N * 4 + 255) / 256) * 256;
}

// ------------------------------------------------------------------ 1. preprocess
// 16 lanes per row; each lane handles D/16 of the row's elements.
template <bool BF16, int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const uint16_t* __restrict__ O, const uint16_t* __restrict__ dO,
                                                      float* __restrict__ Dsum, size_t rows) {
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
  }
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, LPR);
  if (row < rows && sub == 0) Dsum[row] = acc;
}

// ------------------------------------------------------------------ 2. dK, dV
// LDS: Q, dO tiles [64 rows][D] double buffered with XOR-swizzled 16-byte chunks (read row-wise
// with ds_read_b128 and transposed with ds_read_b64_tr_b16; the lane-dependent offsets are
// computed once), then float LSE*log2(e) and D for both buffers.
template <int D>
struct DkdvSmem {
  static constexpr int TILE = kBwdRows * D;
  static constexpr int Q_OFF(int buf) { return buf * 2 * TILE; }
  static constexpr int DO_OFF(int buf) { return buf * 2 * TILE + TILE; }
  static constexpr int F_OFF = 4 * TILE;
  static constexpr size_t BYTES = (size_t)F_OFF * 2 + 2 * 2 * kBwdRows * 4;
};

template <bool BF16, int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Dsum,
    uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, int Hq, int Hkv, int N, int nkb,
    float c /* scale * log2(e) */, float scale) {
  using SM = DkdvSmem<D>;
  constexpr int CH = D / 8, KK = D / 16, DB = D / 32;
  constexpr int NLD = kBwdRows * CH / 256;          // 16-byte chunks per thread per tile
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
  const uint32_t head_bytes = (uint32_t)N * D * 2;
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(K + kv_off, head_bytes);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(V + kv_off, head_bytes);

  // persistent B operands of S = Q K^T and dP = dO V^T: this wave's 32 K and V rows
  i16x8_t kf[KK], vf[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    const uint32_t off = ((uint32_t)(kw + l32) * D + 16 * kk + 8 * g) * 2;
    kf[kk] = __builtin_bit_cast(i16x8_t, buffer_load16(krs, off));
    vf[kk] = __builtin_bit_cast(i16x8_t, buffer_load16(vrs, off));
  }
  wait_all_loads();
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
  // causal: only the first kBwdKeys / kBwdRows query blocks of every head cross the diagonal
  constexpr int kDiag = kBwdKeys / kBwdRows;

  // lane-dependent LDS offsets (16-bit units), loop invariant
  int off_row[KK];                 // A operand rows 32qs + l32, chunk 2kk + g (qs adds 32 rows)
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) off_row[kk] = chunk_index<D>(l32, 2 * kk + g) * 8;
  int off_tr[DB][2];               // transposed reads: rows 4(G16/2) + li/4 (+8), column block db
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int h = 0; h < 2; ++h)
      off_tr[db][h] = elem_index<D>(4 * (G16 >> 1) + (li >> 2) + 8 * h, 32 * db + 16 * (G16 & 1) + 4 * (li & 3));

  uint4 qreg[NLD], doreg[NLD];
  float lse_reg = 0.f, d_reg = 0.f;
  auto block_of = [&](int it, int& h, int& q0) {
    const int hh = it / per_head;
    h = kvh * G + hh;
    q0 = (qstart + it - hh * per_head) * kBwdRows;
  };
  auto load_tile = [&](int it) {
    int h, q0;
    block_of(it, h, q0);
    const size_t q_row0 = ((size_t)b * Hq + h) * (size_t)N;
    const __amdgpu_buffer_rsrc_t qrs = make_rsrc(Q + q_row0 * D, head_bytes);
    const __amdgpu_buffer_rsrc_t ors = make_rsrc(dO + q_row0 * D, head_bytes);
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int cidx = tid + 256 * i;
      const int row = cidx / CH, ch = cidx % CH;
      const uint32_t off = ((uint32_t)(q0 + row) * D + ch * 8) * 2;
      qreg[i] = buffer_load16(qrs, off);
      doreg[i] = buffer_load16(ors, off);
    }
    if (tid < kBwdRows) {
      const int q = q0 + tid;
      lse_reg = q < N ? LSE[q_row0 + q] * kLog2e : 0.f;
      d_reg = q < N ? Dsum[q_row0 + q] : 0.f;
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

  // One query block: S, dP, P, dS, dV, dK.
  auto step = [&](int it, auto mask_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const int buf = it & 1;
    const bool has_next = it + 1 < total;
    if (has_next) load_tile(it + 1);
    int h, q0;
    block_of(it, h, q0);
    const short* Qs = sm + SM::Q_OFF(buf);
    const short* dOs = sm + SM::DO_OFF(buf);
    const float* lse_s = smf + buf * 2 * kBwdRows;
    const float* d_s = lse_s + kBwdRows;
    const int key = kw + l32;
#pragma unroll
    for (int qs = 0; qs < 2; ++qs) {
      // S = Q K^T, dP = dO V^T for rows 32qs .. 32qs+31 of the block
      f32x16_t sacc = f32x16_t{}, dp = f32x16_t{};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const i16x8_t aq = __builtin_bit_cast(i16x8_t, *(const uint4*)(Qs + 32 * qs * D + off_row[kk]));
        const i16x8_t ado = __builtin_bit_cast(i16x8_t, *(const uint4*)(dOs + 32 * qs * D + off_row[kk]));
        sacc = mfma32x32x16<BF16>(aq, kf[kk], sacc);
        dp = mfma32x32x16<BF16>(ado, vf[kk], dp);
      }
      // scheduling hint: the LDS reads of the S/dP operands run two MFMA pairs ahead of their
      // use (mask 0x100 = LDS reads, 0x008 = MFMA); left alone the compiler issues each read
      // right before its MFMA and the single wave per SIMD waits out every LDS latency
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * 2, 0);
#pragma unroll
      for (int i = 0; i < KK; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
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
          float p = __builtin_amdgcn_exp2f(sacc[r] * c - lv[e]);
          if constexpr (MASK) {
            if (key > q0 + qr + e) p = 0.f;
          }
          sacc[r] = p;
          dp[r] = p * (dp[r] - dv4[e]);
        }
      }
      const i16x8_t pb[2] = {pack8<BF16>(sacc, 0), pack8<BF16>(sacc, 8)};
      const i16x8_t sb[2] = {pack8<BF16>(dp, 0), pack8<BF16>(dp, 8)};
      // dV^T += dO^T P ; dK^T += Q^T dS   (k = query rows, slot (g, e) as in the forward)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int rbase = (32 * qs + 16 * t) * D;   // 16 | row offset keeps the swizzle unchanged
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const i16x4_t a0 = ds_read_tr16(dOs + rbase + off_tr[db][0]);
          const i16x4_t a1 = ds_read_tr16(dOs + rbase + off_tr[db][1]);
          const i16x8_t ado = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
          dvacc[db] = mfma32x32x16<BF16>(ado, pb[t], dvacc[db]);
          const i16x4_t b0 = ds_read_tr16(Qs + rbase + off_tr[db][0]);
          const i16x4_t b1 = ds_read_tr16(Qs + rbase + off_tr[db][1]);
          const i16x8_t aq = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
          dkacc[db] = mfma32x32x16<BF16>(aq, sb[t], dkacc[db]);
        }
      }
      // scheduling hint: the transposed reads of dO^T / Q^T run two MFMA pairs ahead
      __builtin_amdgcn_sched_group_barrier(0x100, 4 * 2, 1);
#pragma unroll
      for (int i = 0; i < 2 * DB; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 1);
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 1);
      }
    }
    if (has_next) store_tile(buf ^ 1);
    // one barrier per block: the next tile becomes visible and every wave is done with the
    // buffer the block after overwrites
    __syncthreads();
  };

  if (total > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();
  int it = 0;
  if constexpr (CAUSAL) {
    for (int hh = 0; hh < G; ++hh) {
      const int diag_end = min(hh * per_head + kDiag, (hh + 1) * per_head);
      for (; it < diag_end; ++it) step(it, std::true_type{});
      for (; it < (hh + 1) * per_head; ++it) step(it, std::false_type{});
    }
  } else {
    for (; it < total; ++it) step(it, std::false_type{});
  }

  // epilogue: lane owns key kw + l32; register r holds d = 32db + 8(r/4) + 4g + r%4
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

// ------------------------------------------------------------------ 3. dQ
// LDS per buffer: K tile [64 keys][D] with XOR-swizzled chunks (row reads for S^T and
// transposed reads for dQ^T), V tile [64 keys][D] with rows padded by 16 bytes (row reads).
template <int D>
struct DqSmem {
  static constexpr int KT = kDqKeys * D;
  static constexpr int VSTR = D + 8;
  static constexpr int VT = kDqKeys * VSTR;
  static constexpr int BUF = KT + VT;
  static constexpr size_t BYTES = (size_t)2 * BUF * 2;
};

template <bool BF16, int D, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void bwd_dq_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Dsum,
    uint16_t* __restrict__ dQ, int Hq, int Hkv, int N, int BH, int nqb, float c /* scale * log2(e) */,
    float scale) {
  using SM = DqSmem<D>;
  constexpr int CH = D / 8, KK = D / 16, DB = D / 32, KB = kDqKeys / 32;
  constexpr int NLD = kDqKeys * CH / 256;
  constexpr int VSTR = SM::VSTR;
  extern __shared__ uint4 smem_u4[];
  short* sm = (short*)smem_u4;
  auto Ks = [&](int buf) { return sm + buf * SM::BUF; };
  auto Vs = [&](int buf) { return sm + buf * SM::BUF + SM::KT; };

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, g = lane >> 5, l32 = lane & 31;
  const int G16 = lane >> 4, li = lane & 15;
  const int L = blockIdx.x;
  const int qblk = CAUSAL ? (nqb - 1 - L / BH) : (L / BH);
  const int bh = L % BH;
  const int h = bh % Hq, b = bh / Hq;
  const int kvh = h / (Hq / Hkv);
  const size_t q_row0 = ((size_t)b * Hq + h) * (size_t)N;
  const size_t kv_off = ((size_t)b * Hkv + kvh) * (size_t)N * D;
  const uint32_t head_bytes = (uint32_t)N * D * 2;
  const __amdgpu_buffer_rsrc_t qrs = make_rsrc(Q + q_row0 * D, head_bytes);
  const __amdgpu_buffer_rsrc_t ors = make_rsrc(dO + q_row0 * D, head_bytes);
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(K + kv_off, head_bytes);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(V + kv_off, head_bytes);

  const int q0 = qblk * kDqRows;
  const int qw = q0 + 32 * w;
  const int qrow = qw + l32;
  // B operands for S^T = K Q^T and dP^T = V dO^T: lane holds row qrow, 8 columns 16kk + 8g
  i16x8_t qf[KK], dof[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    const uint32_t off = ((uint32_t)qrow * D + 16 * kk + 8 * g) * 2;
    qf[kk] = __builtin_bit_cast(i16x8_t, buffer_load16(qrs, off));
    dof[kk] = __builtin_bit_cast(i16x8_t, buffer_load16(ors, off));
  }
  // rows past the end: LSE = +inf gives P = 0
  const float lse2 = qrow < N ? LSE[q_row0 + qrow] * kLog2e : INFINITY;
  const float dd = qrow < N ? Dsum[q_row0 + qrow] : 0.f;
  wait_all_loads();

  f32x16_t acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16_t{};

  // lane-dependent K-tile offsets (16-bit units), loop invariant
  int off_row[KK];                 // S^T A operand: rows 32kb + l32, chunk 2kk + g
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) off_row[kk] = chunk_index<D>(l32, 2 * kk + g) * 8;
  int off_tr[DB][2];               // K^T A operand: rows 4(G16/2) + li/4 (+8), column block db
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
      off_tr[db][hh] = elem_index<D>(4 * (G16 >> 1) + (li >> 2) + 8 * hh, 32 * db + 16 * (G16 & 1) + 4 * (li & 3));

  const int kend = CAUSAL ? min(N, q0 + kDqRows) : N;
  const int ntiles = (kend + kDqKeys - 1) / kDqKeys;
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
      *(uint4*)(Ks(buf) + chunk_index<D>(row, ch) * 8) = kreg[i];
      *(uint4*)(Vs(buf) + row * VSTR + ch * 8) = vreg[i];
    }
  };

  auto tile = [&](int j, auto mask_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const int kt0 = j * kDqKeys;
    const bool has_next = j + 1 < ntiles;
    if (has_next) load_tile(kt0 + kDqKeys);
    const bool active = (qw < N) && (!CAUSAL || kt0 <= qw + 31);
    if (active) {
      const short* Kb = Ks(j & 1);
      const short* Vb = Vs(j & 1);
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        // S^T, dP^T for keys 32kb .. 32kb+31 of the tile
        f32x16_t st = f32x16_t{}, dpt = f32x16_t{};
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          const i16x8_t ak = __builtin_bit_cast(i16x8_t, *(const uint4*)(Kb + 32 * kb * D + off_row[kk]));
          const i16x8_t av =
              __builtin_bit_cast(i16x8_t, *(const uint4*)(Vb + (32 * kb + l32) * VSTR + 16 * kk + 8 * g));
          st = mfma32x32x16<BF16>(ak, qf[kk], st);
          dpt = mfma32x32x16<BF16>(av, dof[kk], dpt);
        }
        // dS^T; lane owns query qrow, register r holds key kt0 + 32kb + 8(r/4) + 4g + r%4
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float p = __builtin_amdgcn_exp2f(st[r] * c - lse2);
          if constexpr (MASK) {
            if (kt0 + 32 * kb + 8 * (r >> 2) + 4 * g + (r & 3) > qrow) p = 0.f;
          }
          st[r] = p * (dpt[r] - dd);
        }
        const i16x8_t sb[2] = {pack8<BF16>(st, 0), pack8<BF16>(st, 8)};
        // dQ^T += K^T dS^T: slot (g, e) of half t is key 16t + 8(e/4) + 4g + e%4 (+32kb)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int rbase = (32 * kb + 16 * t) * D;
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const i16x4_t a0 = ds_read_tr16(Kb + rbase + off_tr[db][0]);
            const i16x4_t a1 = ds_read_tr16(Kb + rbase + off_tr[db][1]);
            const i16x8_t ak = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
            acc[db] = mfma32x32x16<BF16>(ak, sb[t], acc[db]);
          }
        }
      }
    }
    if (has_next) store_tile((j + 1) & 1);
    __syncthreads();
  };

  load_tile(0);
  store_tile(0);
  __syncthreads();
  // tiles [0, jmask) are wholly below the diagonal for every wave of the workgroup
  const int jmask = CAUSAL ? min(ntiles, q0 / kDqKeys) : ntiles;
  int j = 0;
  for (; j < jmask; ++j) tile(j, std::false_type{});
  for (; j < ntiles; ++j) tile(j, std::true_type{});

  // epilogue: dQ = scale * dQ^T; register r of block db holds d = 32db + 8(r/4) + 4g + r%4
  if (qrow < N) {
    uint16_t* dqp = dQ + (q_row0 + qrow) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int d0 = 32 * db + 8 * rr + 4 * g;
        uint2 pk;
        pk.x = pack2<BF16>(acc[db][4 * rr + 0] * scale, acc[db][4 * rr + 1] * scale);
        pk.y = pack2<BF16>(acc[db][4 * rr + 2] * scale, acc[db][4 * rr + 3] * scale);
        *(uint2*)(dqp + d0) = pk;
      }
  }
}

// ------------------------------------------------------------------ launchers
template <bool BF16, int D>
static hipError_t launch_pre_t(const void* o, const void* dout, size_t rows, void* workspace, hipStream_t stream) {
  hipLaunchKernelGGL((bwd_pre_kernel<BF16, D>), dim3((unsigned)((rows + 15) / 16)), dim3(256), 0, stream,
                     (const uint16_t*)o, (const uint16_t*)dout, (float*)workspace, rows);
  return hipGetLastError();
}

template <bool BF16, int D, bool CAUSAL>
static hipError_t launch_dkdv_t(const void* q, const void* k, const void* v, const void* dout, const float* lse,
                                void* dk, void* dv, int B, int Hq, int Hkv, int N, float scale, const void* workspace,
                                hipStream_t stream) {
  const int nkb = (N + kBwdKeys - 1) / kBwdKeys;
  auto kern = bwd_dkdv_kernel<BF16, D, CAUSAL>;
  const size_t lds = DkdvSmem<D>::BYTES;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(nkb * B * Hkv), dim3(256), lds, stream, (const uint16_t*)q, (const uint16_t*)k,
                     (const uint16_t*)v, (const uint16_t*)dout, lse, (const float*)workspace, (uint16_t*)dk,
                     (uint16_t*)dv, Hq, Hkv, N, nkb, scale * kLog2e, scale);
  return hipGetLastError();
}

template <bool BF16, int D, bool CAUSAL>
static hipError_t launch_dq_t(const void* q, const void* k, const void* v, const void* dout, const float* lse,
                              void* dq, int B, int Hq, int Hkv, int N, float scale, const void* workspace,
                              hipStream_t stream) {
  const int nqb = (N + kDqRows - 1) / kDqRows;
  const int BH = B * Hq;
  auto kern = bwd_dq_kernel<BF16, D, CAUSAL>;
  const size_t lds = DqSmem<D>::BYTES;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(nqb * BH), dim3(256), lds, stream, (const uint16_t*)q, (const uint16_t*)k,
                     (const uint16_t*)v, (const uint16_t*)dout, lse, (const float*)workspace, (uint16_t*)dq, Hq, Hkv,
                     N, BH, nqb, scale * kLog2e, scale);
  return hipGetLastError();
}

hipError_t launch_bwd_pre(const void* o, const void* dout, int B, int Hq, int N, int d, bool bf16, void* workspace,
                          hipStream_t stream) {
  const size_t rows = (size_t)B * Hq * N;
  if (bf16) return d == 128 ? launch_pre_t<true, 128>(o, dout, rows, workspace, stream)
                            : launch_pre_t<true, 64>(o, dout, rows, workspace, stream);
  return d == 128 ? launch_pre_t<false, 128>(o, dout, rows, workspace, stream)
                  : launch_pre_t<false, 64>(o, dout, rows, workspace, stream);
}

#define EAO_DISPATCH(FN, ...)                                                                 \
  if (bf16) {                                                                                 \
    if (d == 128) {                                                                           \
      if (causal) return FN<true, 128, true>(__VA_ARGS__);                                    \
      return FN<true, 128, false>(__VA_ARGS__);                                               \
    }                                                                                         \
    if (causal) return FN<true, 64, true>(__VA_ARGS__);                                       \
    return FN<true, 64, false>(__VA_ARGS__);                                                  \
  }                                                                                           \
  if (d == 128) {                                                                             \
    if (causal) return FN<false, 128, true>(__VA_ARGS__);                                     \
    return FN<false, 128, false>(__VA_ARGS__);                                                \
  }                                                                                           \
  if (causal) return FN<false, 64, true>(__VA_ARGS__);                                        \
  return FN<false, 64, false>(__VA_ARGS__);

hipError_t launch_bwd_dkdv(const void* q, const void* k, const void* v, const void* dout, const float* lse, void* dk,
                           void* dv, int B, int Hq, int Hkv, int N, int d, bool causal, float scale, bool bf16,
                           const void* workspace, hipStream_t stream) {
  EAO_DISPATCH(launch_dkdv_t, q, k, v, dout, lse, dk, dv, B, Hq, Hkv, N, scale, workspace, stream)
}

hipError_t launch_bwd_dq(const void* q, const void* k, const void* v, const void* dout, const float* lse, void* dq,
                         int B, int Hq, int Hkv, int N, int d, bool causal, float scale, bool bf16,
                         const void* workspace, hipStream_t stream) {
  EAO_DISPATCH(launch_dq_t, q, k, v, dout, lse, dq, B, Hq, Hkv, N, scale, workspace, stream)
}
#undef EAO_DISPATCH

}  // namespace eao
