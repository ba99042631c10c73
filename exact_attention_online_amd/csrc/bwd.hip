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
//   1. bwd_pre: per query row -D = -rowsum(dO * O) and LSE * log2(e), in the caller's workspace.
//   2. bwd_dkdv: one workgroup of 8 waves per (batch, K/V head, block of 128 keys), in two
//      roles over the same four quarters of 32 keys (one wave of each role per SIMD).  A "P
//      wave" keeps its keys' K fragments and dV^T in registers, a "dS wave" their V fragments
//      and dK^T.  The workgroup walks every query head of the K/V head's group and every tile
//      of 64 query rows (causal: from the diagonal on), so dK and dV are summed over the group
//      in registers.  The row-major tiles of Q and dO and the rows' LSE2 and -D go straight
//      from HBM into triple-buffered LDS (direct buffer -> LDS loads, two tiles ahead).  Per
//      tile (a lane owns one key column of every accumulator):
//        P wave:  P = exp2(S * scale * log2e - LSE * log2e) from the S computed one tile earlier
//                 (causal mask on the diagonal tiles only), rounded to the input type and
//                 passed to the partner through LDS;  dV^T += dO^T P;  S = Q K^T of the next tile
//        dS wave: dP - D = dO V^T accumulated from -D;  dS = P (dP - D);  dK^T += Q^T dS
//      Q and dO are read as rows (ds_read_b128), dO^T and Q^T from the same tiles through
//      ds_read_b64_tr_b16.  Computing S a tile ahead lets the P wave's exponentials run while
//      the dS wave's dP MFMAs occupy the matrix core.  Two contractions per wave (three MFMA
//      groups for the P wave) keep each wave under 256 registers, so two waves share a SIMD.
//   3. bwd_dq: one workgroup of 8 waves per (batch, query head, block of 256 query rows),
//      shaped like the forward: a lane owns one query row, so LSE and D are one register each.
//      Per key tile of 64:
//        S^T = K Q^T, dP^T = V dO^T, dS^T = P^T * (dP^T - D), dQ^T += K^T dS^T,
//      with dS^T fed from the accumulator into the last MFMA (k relabelled as in the forward)
//      and K^T read from the row-major K tile through ds_read_b64_tr_b16; dQ = scale * dQ^T is
//      written once at the end.
// Splitting dQ off costs two extra contractions (S and dP are recomputed) but replaces the
// fp32 atomic accumulation of dQ, whose ordered completion stalled the loads of the
// key-stationary kernel, with plain register accumulation.
//
// Keys or query rows past N read as zeros (bounds-checked buffer loads).  Zero K/V rows and
// zero Q/dO/D rows make every contribution that crosses the end of the sequence vanish exactly,
// so only the causal diagonal (and, with a sliding window, the band's edges) is masked.
//
// Variants of the same kernels: VARLEN (sequences packed without padding, offsets from
// cu_seqlens) and EXT (sliding window and ALiBi bias), described at the kernels.
#include <algorithm>
#include <type_traits>

#include "common.hpp"

namespace eao {

constexpr int kBwdKeys = 128;   // keys per dK/dV workgroup (32 per wave)
constexpr int kBwdRows = 64;    // query rows per dK/dV step (one tile)
constexpr int kDqRows = 256;    // query rows per dQ workgroup (8 waves x 32; 4 x 32 on small grids)
constexpr int kDqKeys = 64;     // keys per dQ step

// Workspace layout (bytes), Npad = 64 * ceil(N / 64), A = roundup(B * Hq * Npad * 4, 256):
//   [0, A)           -D    float  [B*Hq][Npad]   -rowsum(dO * O); 0 past N
//   [A, 2A)          LSE2  float  [B*Hq][Npad]   LSE * log2(e); +inf past N
//   [2A, ...)        fp32 dK/dV shares of a split dK/dV phase (dkdv_splits > 1)
// Row range of sequence b in a packed variable-length batch: cu_seqlens entries clamped to
// [0, T] and made non-decreasing, and the length capped at the workspace rows per head (npad),
// so that a malformed array cannot send a kernel outside its buffers.
struct SeqRange {
  int s0, n;
};
__device__ __forceinline__ SeqRange seq_range(const int* __restrict__ cu, int b, int T, int npad) {
  const int s0 = min(max(cu[b], 0), T);
  const int s1 = min(max(cu[b + 1], s0), T);
  return SeqRange{s0, min(s1 - s0, npad)};
}

struct BwdWs {
  float* dsum;
  float* lse2;
  float* part;      // fp32 dK/dV shares of a split dK/dV phase (dkdv_splits > 1)
  int npad;
};

static BwdWs bwd_ws(void* workspace, int B, int Hq, int N) {
  BwdWs w;
  w.npad = (N + kBwdRows - 1) / kBwdRows * kBwdRows;
  const size_t a = ((size_t)B * Hq * w.npad * 4 + 255) / 256 * 256;
  char* base = (char*)workspace;
  w.dsum = (float*)base;
  w.lse2 = (float*)(base + a);
  w.part = (float*)(base + 2 * a);
  return w;
}

// Splits of the dK/dV phase (dense layout).  The grid has one workgroup per (batch, K/V head,
// block of 128 keys), each walking the G query heads of its group; with few K/V heads and a
// short sequence it leaves most compute units idle.  Below one workgroup per CU the (query head,
// query tile) steps of every key block are cut into up to 2G ranges (about two workgroups per
// CU in all), each range's dK/dV share is kept in fp32 in the workspace and a second kernel adds
// the shares in a fixed order: no atomics, deterministic.
int dkdv_splits(int B, int Hq, int Hkv, int N) {
  const int G = Hq / Hkv;
  const long long wg = (long long)B * Hkv * ((N + kBwdKeys - 1) / kBwdKeys);
  if (G < 2 || wg >= kNumCUs) return 1;
  return (int)std::min<long long>((2 * kNumCUs + wg - 1) / wg, 2 * G);
}

size_t bwd_workspace_bytes(int B, int Hq, int Hkv, int N, int d, bool dense) {
  const size_t npad = (size_t)(N + kBwdRows - 1) / kBwdRows * kBwdRows;
  const size_t a = ((size_t)B * Hq * npad * 4 + 255) / 256 * 256;
  size_t bytes = 2 * a;
  const int ns = dense ? dkdv_splits(B, Hq, Hkv, N) : 1;
  if (ns > 1) bytes += (size_t)ns * 2 * B * Hkv * N * d * 4;
  return bytes;
}

// ------------------------------------------------------------------ 1. preprocess
// One workgroup of 256 threads per (batch * query head, 64-row tile): -D and LSE2 of the tile's
// rows.  Thread t reads the 16-byte chunks t + 256 i of the tile's O and dO rows, so the D / 8
// threads of one row are consecutive lanes and one row sum is a shuffle reduction.  Rows past
// N get -D = 0 and LSE2 = +inf.
//
// VARLEN: sequences packed without padding, O/dO [Hq,T,d], LSE [Hq,T] (T = N_in rows),
// sequence b = rows cu_seqlens[b] .. cu_seqlens[b+1]-1; the workspace keeps the [B*H][npad]
// layout with npad from the longest sequence, and tiles past a sequence's end are not written.
template <bool BF16, int D, bool VARLEN = false>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const uint16_t* __restrict__ O, const uint16_t* __restrict__ dO,
                                                      const float* __restrict__ LSE, float* __restrict__ Dsum,
                                                      float* __restrict__ Lse2, int N_in, int npad, int Hq,
                                                      const int* __restrict__ cu_seqlens) {
  constexpr int CH = D / 8;                  // 16-byte chunks per row
  constexpr int CPT = kBwdRows * CH / 256;   // chunks per thread per tile
  const int ntile = npad / kBwdRows;
  const int tid = threadIdx.x;
  const int bh = blockIdx.x / ntile, tile = blockIdx.x % ntile;
  int N = N_in;
  size_t row0 = (size_t)bh * N_in;             // first row of the head (sequence) in O, dO, LSE
  if constexpr (VARLEN) {
    const SeqRange sr = seq_range(cu_seqlens, bh / Hq, N_in, npad);
    if (tile * kBwdRows >= sr.n) return;
    N = sr.n;
    row0 = (size_t)(bh % Hq) * N_in + sr.s0;
  }
  const size_t base = (row0 + (size_t)tile * kBwdRows) * D;
  uint4 ov[CPT], dv[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int ci = tid + 256 * i, row = ci / CH, ch = ci % CH;
    ov[i] = dv[i] = uint4{0, 0, 0, 0};
    if (tile * kBwdRows + row < N) {
      ov[i] = *(const uint4*)(O + base + (size_t)row * D + 8 * ch);
      dv[i] = *(const uint4*)(dO + base + (size_t)row * D + 8 * ch);
    }
  }
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int ci = tid + 256 * i, row = ci / CH, ch = ci % CH;
    const int q = tile * kBwdRows + row;
    const uint16_t* o16 = (const uint16_t*)&ov[i];
    const uint16_t* d16 = (const uint16_t*)&dv[i];
    float acc = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc += to_float<BF16>(o16[e]) * to_float<BF16>(d16[e]);
#pragma unroll
    for (int off = CH / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, CH);
    if (ch == 0) {
      const size_t r = (size_t)bh * npad + q;
      Dsum[r] = q < N ? -acc : 0.f;
      Lse2[r] = q < N ? LSE[row0 + q] * kLog2e : INFINITY;
    }
  }
}

// One gradient row from an accumulator whose register r of block db holds column
// 32db + 8(r/4) + 4g + r%4, times f: stored as float (out32) or rounded to the input type.
// `elem` is the row's first element; the row is D = 32 * DB values.
template <bool BF16, int DB>
__device__ __forceinline__ void store_row(void* __restrict__ base, size_t elem, const f32x16_t (&acc)[DB], float f,
                                          int g, int out32) {
  if (out32) {
    float* dst = (float*)base + elem;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int d0 = 32 * db + 8 * rr + 4 * g;
        *(float4*)(dst + d0) = float4{acc[db][4 * rr + 0] * f, acc[db][4 * rr + 1] * f, acc[db][4 * rr + 2] * f,
                                      acc[db][4 * rr + 3] * f};
      }
  } else {
    uint16_t* dst = (uint16_t*)base + elem;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int d0 = 32 * db + 8 * rr + 4 * g;
        uint2 pk;
        pk.x = pack2<BF16>(acc[db][4 * rr + 0] * f, acc[db][4 * rr + 1] * f);
        pk.y = pack2<BF16>(acc[db][4 * rr + 2] * f, acc[db][4 * rr + 3] * f);
        *(uint2*)(dst + d0) = pk;
      }
  }
}

// ------------------------------------------------------------------ 2. dK, dV
// One workgroup of 8 waves per (batch, K/V head, block of 128 keys).  The waves come in two
// roles over the same four quarters of 32 keys, one wave of each role per SIMD:
//   P waves (0-3):  hold K and dV^T of their 32 keys; per query tile P = exp2(S c - LSE2) from
//                   the S computed during the previous tile (causal mask on the diagonal tiles),
//                   P rounded to the input type and handed to the partner wave through LDS,
//                   then dV^T += dO^T P and S = Q K^T of the next tile;
//   dS waves (4-7): hold V and dK^T; dP - D = dO V^T accumulated from -D, then, with the
//                   partner's P, dS = P (dP - D) and dK^T += Q^T dS.
// Each wave needs fewer than 256 registers, so two waves share each SIMD; with S one tile
// ahead, the P wave's exponentials run while the dS wave's dP MFMAs use the matrix core, and
// the dS wave's products run beside the P wave's MFMAs.  Per step (one 64-row query tile) the
// tile [Q | dO] ([64 rows][D] each, chunks XOR-swizzled by swz) and LSE2 and -D of the 64 rows
// go straight from HBM into triple-buffered LDS (direct buffer -> LDS loads two steps ahead,
// each buffer a distinct LDS object).  Q and dO are read as 16-byte rows (A operands of S and
// dP), Q^T and dO^T through transposed reads of the same tiles (A operands of dK^T and dV^T).
// Two barriers per step: A (P of this tile written, next tile landed) and X (this tile's
// buffer free for the loads of the tile three steps on).  Each half of a step holds the same
// matrix work: before A the P wave's dV^T MFMAs (its own P needs no exchange) beside the dS
// wave's dP MFMAs, after A the P wave's S MFMAs of the next tile beside the dS wave's dK^T.
// VARLEN: packed sequences as in bwd_pre_kernel (K/V/dK/dV [Hkv,T,d], Q/dO [Hq,T,d]); a key block
// past its sequence's end exits at once.
// EXT: the sliding window and ALiBi bias of the forward with the same flag (key j visible to query
// i only if i - j < window, and without the causal mask also j - i < window; score (i, j) of
// query head h gets -slopes[h] |i - j| after the softmax scale).  The bias is constant in Q and
// K, so the gradients keep their form and only the recomputed P changes: every query tile in
// the band of the key block takes the masked path with the bias, tiles outside it are skipped.
template <bool BF16, int D, bool CAUSAL, bool VARLEN = false, bool EXT = false, bool ALIBI = false>
__global__ __launch_bounds__(512, 1) void bwd_dkdv_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ Dneg, const float* __restrict__ Lse2,
    void* __restrict__ dK, void* __restrict__ dV, int Hq, int Hkv, int N_in, int npad, int nkb,
    float c /* scale * log2(e) */, float scale, const int* __restrict__ cu_seqlens, int window,
    const float* __restrict__ slopes, int out32, float* __restrict__ part, int nsplit) {
  constexpr int CH = D / 8, KK = D / 16, DB = D / 32;
  constexpr int NW = 8;                              // waves per workgroup
  constexpr int TILE = kBwdRows * D;                 // 16-bit elements per tile
  constexpr int PIECES = TILE * 2 / 1024;            // 1 KB direct-load pieces per tile
  static_assert(PIECES % NW == 0, "each wave moves the same number of pieces of every tile");
  constexpr int PW = PIECES / NW;
  // [Q | dO] of one query tile, three buffers
  __shared__ __attribute__((aligned(1024))) short qd0[2 * TILE];
  __shared__ __attribute__((aligned(1024))) short qd1[2 * TILE];
  __shared__ __attribute__((aligned(1024))) short qd2[2 * TILE];
  // [LSE2 of the 64 rows | unused][-D of the 64 rows | unused], 1 KB each
  __shared__ __attribute__((aligned(1024))) float st0[512];
  __shared__ __attribute__((aligned(1024))) float st1[512];
  __shared__ __attribute__((aligned(1024))) float st2[512];
  // P of each key quarter: [quarter][slot 2 * half + t][lane], 16 bytes each
  __shared__ __attribute__((aligned(1024))) uint4 pex[4 * 4 * 64];
  auto QD = [&](auto par) __attribute__((always_inline)) -> short* {
    if constexpr (decltype(par)::value == 0) return qd0;
    else if constexpr (decltype(par)::value == 1) return qd1;
    else return qd2;
  };
  auto ST = [&](auto par) __attribute__((always_inline)) -> float* {
    if constexpr (decltype(par)::value == 0) return st0;
    else if constexpr (decltype(par)::value == 1) return st1;
    else return st2;
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, g = lane >> 5, l32 = lane & 31;
  const int wu = __builtin_amdgcn_readfirstlane(w);            // the same, known to be uniform
  const int role = wu >> 2;                                      // 0: P wave, 1: dS wave
  const int kq = w & 3;                                         // key quarter
  const int G = Hq / Hkv;
  // key block major: under causal masking the first key blocks see the most query rows, so
  // the heaviest workgroups of every head start first
  // split sp of nsplit of this key block's steps (adjacent workgroups, sharing the block's K and
  // V in L2; nsplit = 1 except for small grouped-query grids, see dkdv_splits)
  const int sp = (int)blockIdx.x % nsplit;
  const int L = (int)blockIdx.x / nsplit;
  const int BHkv = gridDim.x / (nkb * nsplit);
  // packed sequences: the same order, sequence by sequence (all blocks of sequence b's heads
  // before sequence b + 1), so that the workgroups in flight share their sequence's query tiles
  // in L2 as the workgroups of one batch do
  const int kblk = VARLEN ? (L % (Hkv * nkb)) / Hkv : L / BHkv;
  const int bkv = VARLEN ? (L / (Hkv * nkb)) * Hkv + L % Hkv : L % BHkv;
  const int b = bkv / Hkv, kvh = bkv % Hkv;
  const int k0 = kblk * kBwdKeys;
  const int kw = k0 + 32 * kq;                      // this wave's first key
  int N = N_in, s0 = 0;
  if constexpr (VARLEN) {
    const SeqRange sr = seq_range(cu_seqlens, b, N_in, npad);
    if (k0 >= sr.n) return;                         // the whole workgroup: no barrier reached
    N = sr.n;
    s0 = sr.s0;
  }
  // first row of a head (of this sequence) in the [B,H,N,d] or packed [H,T,d] tensors
  auto head_row0 = [&](int bh_b, int hh) __attribute__((always_inline)) -> size_t {
    if constexpr (VARLEN) return (size_t)hh * N_in + s0;
    else return (size_t)bh_b * N;
  };
  const size_t kv_off = head_row0(b * Hkv + kvh, kvh) * D;
  const uint32_t head_bytes = (uint32_t)N * D * 2;

  // persistent B operands: K rows (P waves) or V rows (dS waves) of the wave's 32 keys
  i16x8_t kvf[KK];
  {
    const __amdgpu_buffer_rsrc_t frs = make_rsrc((role == 0 ? K : V) + kv_off, head_bytes);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      kvf[kk] = __builtin_bit_cast(i16x8_t, buffer_load16(frs, ((uint32_t)(kw + l32) * D + 16 * kk + 8 * g) * 2));
  }
  wait_all_loads();
  // dV^T (P waves) or dK^T (dS waves)
  f32x16_t acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16_t{};

  const int nqb = (N + kBwdRows - 1) / kBwdRows;   // query tiles of the sequence
  // window (0: none; a window of N or more sees everything, so it is capped at N)
  const int W = (EXT && window > 0) ? min(window, N) : 0;
  // query tiles [qstart, qend) hold every row that sees a key of the block
  int qstart = CAUSAL ? (k0 / kBwdRows) : 0;
  int qend = nqb;
  if (W > 0) {
    if (!CAUSAL) qstart = max(0, k0 - W + 1) / kBwdRows;
    qend = min(nqb, (k0 + kBwdKeys + W - 2) / kBwdRows + 1);
  }
  const int per_head = qend - qstart;
  const int total = G * per_head;
  // this workgroup's steps [it0, it1) of the block's G * per_head (query head, query tile) steps
  const int it0 = (int)((long long)total * sp / nsplit);
  const int it1 = (int)((long long)total * (sp + 1) / nsplit);
  // causal: only the first kBwdKeys / kBwdRows query blocks of every head cross the diagonal
  constexpr int kDiag = kBwdKeys / kBwdRows;

  // loop-invariant offsets.  Reads (16-bit units): Q / dO rows 32qs + l32 at chunk 2kk + g;
  // transposed reads (tr_off) for Q^T and dO^T.  Direct loads (bytes): piece NW i + w of a
  // tile, lane l -> LDS chunk 64(NW i + w) + l, fetched from the chunk the swizzle puts there.
  int off_row[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) off_row[kk] = chunk_index<D>(l32, 2 * kk + g) * 8;
  int off_tr[DB][2];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) off_tr[db][hh] = tr_off<D>(lane, db, hh);
  // (piece NW i + w lies 64 NW i / CH rows after piece w, a multiple of the swizzle's period, so
  // its source is dma_qd plus a uniform offset)
  static_assert((64 * NW / CH) % 16 == 0, "pieces of one wave keep the row swizzle");
  uint32_t dma_qd;
  {
    const int pch = 64 * w + lane;
    const int r = pch / CH, cc = pch % CH;
    dma_qd = ((uint32_t)r * D + ((cc ^ swz<D>(r)) << 3)) * 2;
  }

  // Loader state: the block that the next call of load_next fetches (query head ld_hh of the
  // group, rows ld_q0 ..), and buffer descriptors over that head's Q, dO and statistics, rebuilt
  // only when the head changes.
  const int it0_tile = per_head > 0 ? it0 % per_head : 0;
  const int it0_hh = per_head > 0 ? min(it0 / per_head, G - 1) : 0;
  int ld_hh = it0_hh;
  int ld_q0 = (qstart + it0_tile) * kBwdRows, ld_left = per_head - it0_tile;
  __amdgpu_buffer_rsrc_t qrs, ors, srs;
  auto head_rsrcs = [&]() __attribute__((always_inline)) {
    const size_t bhq = (size_t)b * Hq + kvh * G + ld_hh;
    const size_t qoff = head_row0((int)bhq, kvh * G + ld_hh) * D;
    qrs = make_rsrc(Q + qoff, head_bytes);
    ors = make_rsrc(dO + qoff, head_bytes);
    // LSE2 (wave 0) or -D (wave 1) of the head's rows
    srs = make_rsrc((wu == 0 ? Lse2 : Dneg) + bhq * npad, (uint32_t)npad * 4);
  };
  head_rsrcs();
  // direct loads of the loader's block into buffer `par` (two tiles, and the 64 rows' LSE2 and
  // -D from waves 0 and 1, whose lanes 16-63 fetch rows that are never read), then advance the
  // loader; after the last block it stays there, so the last steps reload it into idle buffers
  // instead of branching around the loads
  auto load_next = [&](auto par) __attribute__((always_inline)) {
    short* qd = QD(par);
    const uint32_t off = (uint32_t)ld_q0 * D * 2;
    if (wu < 2) buffer_load16_lds(srs, (short*)(ST(par) + 256 * wu), 16 * lane + (uint32_t)ld_q0 * 4);
#pragma unroll
    for (int i = 0; i < PW; ++i) {
      const int piece = NW * i + wu;
      const uint32_t soff = off + (uint32_t)i * (64 * NW / CH) * D * 2;
      buffer_load16_lds(qrs, qd + 512 * piece, dma_qd, soff);
      buffer_load16_lds(ors, qd + TILE + 512 * piece, dma_qd, soff);
    }
    if (ld_left > 1) {
      --ld_left;
      ld_q0 += kBwdRows;
    } else if (ld_hh + 1 < G) {
      ++ld_hh;
      ld_q0 = qstart * kBwdRows;
      ld_left = per_head;
      head_rsrcs();
    }
  };
  // wait until at most one step's loads (the newest) are in flight: the next tile has landed
  auto wait_but_one_step = [&]() __attribute__((always_inline)) {
    if (wu < 2) wait_vmem<2 * PW + 1>();
    else wait_vmem<2 * PW>();
  };

  // Compute cursor: query head cu_hh of the group and tile cu_t of the head for the current step.
  int cu_hh = it0_hh, cu_t = it0_tile;

  // S = Q K^T of the tile in buffer `par` (P waves): rows 0-31 and 32-63; a lane owns key
  // kw + l32, register r holds row 32qs + 8(r/4) + 4g + r%4
  f32x16_t s[2];
  auto compute_s = [&](auto par) __attribute__((always_inline)) {
    const short* qd = QD(par);
    s[0] = f32x16_t{};
    s[1] = f32x16_t{};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
#pragma unroll
      for (int qs = 0; qs < 2; ++qs) {
        const i16x8_t a = __builtin_bit_cast(i16x8_t, *(const uint4*)(qd + 32 * qs * D + off_row[kk]));
        s[qs] = mfma32x32x16<BF16>(a, kvf[kk], s[qs]);
      }
  };
  // P = exp2(S c - LSE2) in place (P waves); MODE 0 no mask, 1 masked (causal diagonal; EXT:
  // window, causal and bias), 2 (EXT) bias only, for tiles wholly inside the band
  auto probs = [&](const float* st, int q0, float ab2, auto mode_tag) __attribute__((always_inline)) {
    constexpr int MODE = (int)decltype(mode_tag)::value;
    constexpr bool MASK = MODE == 1;
    const int key = kw + l32;
#pragma unroll
    for (int qs = 0; qs < 2; ++qs) {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const float4 l4 = *(const float4*)(st + 32 * qs + 8 * rr + 4 * g);
        const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * rr + e;
          float p;
          if constexpr (EXT && MODE != 0) {
            const int diff = q0 + 32 * qs + 8 * rr + 4 * g + e - key;   // query - key
            float x = s[qs][r] * c - lv[e];
            if constexpr (ALIBI) x = __builtin_fmaf(__builtin_fabsf((float)diff), ab2, x);
            p = __builtin_amdgcn_exp2f(x);
            if constexpr (MASK) {
              const bool vis = (CAUSAL ? diff >= 0 : (W == 0 || diff > -W)) && (W == 0 || diff < W);
              if (!vis) p = 0.f;
            }
          } else {
            p = __builtin_amdgcn_exp2f(s[qs][r] * c - lv[e]);
            if constexpr (MASK) {
              if (key > q0 + 32 * qs + 8 * rr + 4 * g + e) p = 0.f;
            }
          }
          s[qs][r] = p;
        }
      }
    }
  };

  // One query tile in buffer `par` (the loads of the tile two steps on go into buffer `par` + 2),
  // as a P wave and as a dS wave.  The roles run separate loops with the same barriers, so each
  // keeps only its own values in registers.
  auto p_step = [&](auto par) __attribute__((always_inline)) {
    using Next = std::integral_constant<int, (decltype(par)::value + 1) % 3>;
    using Far = std::integral_constant<int, (decltype(par)::value + 2) % 3>;
    load_next(Far{});
    const short* qd = QD(par);
    const float* st = ST(par);
    // ---- P of this tile (S computed during the previous step)
    const int q0 = (qstart + cu_t) * kBwdRows;
    if constexpr (EXT) {
      const int dmin = q0 - (k0 + kBwdKeys - 1), dmax = q0 + kBwdRows - 1 - k0;   // query - key
      const bool inside = (CAUSAL ? dmin >= 0 : (W == 0 || dmin > -W)) && (W == 0 || dmax < W);
      const float ab2 = ALIBI ? -slopes[kvh * G + cu_hh] * kLog2e : 0.f;
      // two tile kinds: masked, and (inside the band) bias-only with ALiBi or plain without
      if (!inside) probs(st, q0, ab2, std::integral_constant<int, 1>{});
      else probs(st, q0, ab2, std::integral_constant<int, ALIBI ? 2 : 0>{});
    } else if constexpr (CAUSAL) {
      if (cu_t < kDiag) probs(st, q0, 0.f, std::integral_constant<int, 1>{});
      else probs(st, q0, 0.f, std::integral_constant<int, 0>{});
    } else {
      probs(st, q0, 0.f, std::integral_constant<int, 0>{});
    }
    // rounded to the input type: B operand of dV^T and the partner's dS; P exchange slots
    // (16-byte units) [quarter][2 * half + t][lane]
    uint4* px = pex + kq * 256 + lane;
    i16x8_t pb[2][2];
#pragma unroll
    for (int qs = 0; qs < 2; ++qs)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        pb[qs][t] = pack8<BF16>(s[qs], 8 * t);
        px[64 * (2 * qs + t)] = __builtin_bit_cast(uint4, pb[qs][t]);
      }
    // ---- dV^T += dO^T P (slot (g, e) of half t is row 32qs + 16t + 8(e/4) + 4g + e%4): this
    // tile's dO has been visible since the previous barrier A
    const short* tdo = qd + TILE;
#pragma unroll
    for (int qs = 0; qs < 2; ++qs)
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const i16x8_t a = read_tr8(tdo + (32 * qs + 16 * t) * D, off_tr[db]);
          acc[db] = mfma32x32x16<BF16>(a, pb[qs][t], acc[db]);
        }
    // scheduling: LDS reads a few ahead of their MFMAs (0x100 = LDS reads, 0x008 = MFMA)
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int i = 0; i < 4 * DB; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    wait_but_one_step();
    lds_barrier();   // A: P is visible to the dS waves, the next tile to every wave
    // ---- S of the next tile (past the workgroup's last step it reads a reloaded block and the
    // result is never used)
    compute_s(Next{});
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
    for (int i = 0; i < 2 * KK; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    lds_barrier();   // X: every wave is done with this tile's buffers (and the P exchange)
    if (cu_t + 1 < per_head) {
      ++cu_t;
    } else {
      ++cu_hh;
      cu_t = 0;
    }
  };
  auto ds_step = [&](auto par) __attribute__((always_inline)) {
    using Far = std::integral_constant<int, (decltype(par)::value + 2) % 3>;
    load_next(Far{});
    const short* qd = QD(par);
    const float* st = ST(par);
    // ---- dP - D = dO V^T accumulated from -D (same layout as S)
    f32x16_t dp[2];
#pragma unroll
    for (int qs = 0; qs < 2; ++qs)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const float4 d4 = *(const float4*)(st + 256 + 32 * qs + 8 * rr + 4 * g);
        dp[qs][4 * rr + 0] = d4.x;
        dp[qs][4 * rr + 1] = d4.y;
        dp[qs][4 * rr + 2] = d4.z;
        dp[qs][4 * rr + 3] = d4.w;
      }
    const short* dos = qd + TILE;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
#pragma unroll
      for (int qs = 0; qs < 2; ++qs) {
        const i16x8_t a = __builtin_bit_cast(i16x8_t, *(const uint4*)(dos + 32 * qs * D + off_row[kk]));
        dp[qs] = mfma32x32x16<BF16>(a, kvf[kk], dp[qs]);
      }
    wait_but_one_step();
    lds_barrier();   // A: the partner's P has been written
    // ---- dS = P (dP - D), packed as the B operand of dK^T
    const uint4* px = pex + kq * 256 + lane;
    i16x8_t sb[2][2];
#pragma unroll
    for (int qs = 0; qs < 2; ++qs)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
        const u32x4_t pw = __builtin_bit_cast(u32x4_t, px[64 * (2 * qs + t)]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 8 * t + 2 * e;
          dp[qs][r] *= lo_to_float<BF16>(pw[e]);
          dp[qs][r + 1] *= hi_to_float<BF16>(pw[e]);
        }
        sb[qs][t] = pack8<BF16>(dp[qs], 8 * t);
      }
    // ---- dK^T += Q^T dS
#pragma unroll
    for (int qs = 0; qs < 2; ++qs)
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const i16x8_t a = read_tr8(qd + (32 * qs + 16 * t) * D, off_tr[db]);
          acc[db] = mfma32x32x16<BF16>(a, sb[qs][t], acc[db]);
        }
    __builtin_amdgcn_sched_group_barrier(0x100, 4 + 4, 0);
#pragma unroll
    for (int i = 0; i < 4 * DB; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    lds_barrier();   // X
  };
  // steps [it0, it1), step it0 in buffer 0
  auto run = [&](auto stepf) __attribute__((always_inline)) {
    using B0 = std::integral_constant<int, 0>;
    using B1 = std::integral_constant<int, 1>;
    using B2 = std::integral_constant<int, 2>;
    int it = it0;
    for (; it + 3 <= it1; it += 3) {
      stepf(B0{});
      stepf(B1{});
      stepf(B2{});
    }
    if (it < it1) {
      stepf(B0{});
      ++it;
    }
    if (it < it1) stepf(B1{});
  };

  if (it1 > it0) {
    load_next(std::integral_constant<int, 0>{});
    load_next(std::integral_constant<int, 1>{});
    wait_but_one_step();
    lds_barrier();
    if (role == 0) {
      compute_s(std::integral_constant<int, 0>{});
      run(p_step);
    } else {
      run(ds_step);
    }
  }

  // epilogue: lane owns key kw + l32; register r holds d = 32db + 8(r/4) + 4g + r%4
  const int key = kw + l32;
  if (key < N) {
    const float f = role == 0 ? 1.f : scale;
    if (part != nullptr) {
      // split: this workgroup's share in fp32, [split][dV, dK][B * Hkv * N][D]; summed in a
      // fixed order by bwd_dkdv_sum_kernel
      const size_t plane = (size_t)BHkv * N * D;
      store_row<BF16, DB>(part + (2 * (size_t)sp + role) * plane, kv_off + (size_t)key * D, acc, f, g, 1);
    } else {
      store_row<BF16, DB>(role == 0 ? dV : dK, kv_off + (size_t)key * D, acc, f, g, out32);
    }
  }
}

// dK, dV = the sum of the nsplit fp32 shares [split][dV, dK][n] (n = B * Hkv * N * D), added in
// split order (deterministic), stored as float (out32) or rounded to the input type.
template <bool BF16>
__global__ __launch_bounds__(256) void bwd_dkdv_sum_kernel(const float* __restrict__ part, void* __restrict__ dK,
                                                           void* __restrict__ dV, size_t n4, int nsplit, int out32) {
  const float4* p4 = (const float4*)part;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < 2 * n4; i += (size_t)gridDim.x * 256) {
    const int role = i >= n4 ? 1 : 0;
    const size_t j = i - (size_t)role * n4;
    float4 a = p4[(size_t)role * n4 + j];
    for (int s = 1; s < nsplit; ++s) {
      const float4 b = p4[(2 * (size_t)s + role) * n4 + j];
      a.x += b.x;
      a.y += b.y;
      a.z += b.z;
      a.w += b.w;
    }
    void* out = role == 0 ? dV : dK;
    if (out32) {
      ((float4*)out)[j] = a;
    } else {
      ((uint2*)out)[j] = uint2{pack2<BF16>(a.x, a.y), pack2<BF16>(a.z, a.w)};
    }
  }
}

// ------------------------------------------------------------------ 3. dQ
// One workgroup of 8 waves per (batch, query head, block of 256 query rows); a wave owns 32
// rows (two waves per SIMD).  When 256-row blocks would give the CUs fewer than two workgroups
// each (dense layout, no window or bias), 4 waves and 128 rows, twice the workgroups; a row's
// arithmetic is the same either way.  Per key tile of 64, the tiles [K | V] ([64][D], chunks
// swizzled by swz) in double-buffered LDS (two distinct LDS objects), filled by direct
// buffer -> LDS loads.  K and V are read as 16-byte rows (A operands of S^T and dP^T), K^T
// through ds_read_b64_tr_b16 of the same K tile (A operand of dQ^T).
// VARLEN: packed sequences as in bwd_pre_kernel; a query block past its sequence's end exits at
// once.  EXT: window and ALiBi as in the dK/dV kernel; key tiles outside the block's band are
// skipped and every other tile takes the masked path with the bias.
template <bool BF16, int D, bool CAUSAL, bool VARLEN = false, bool EXT = false, int ROWS = kDqRows,
          bool ALIBI = false>
__global__ __launch_bounds__(ROWS * 2, 512 / (ROWS * 2)) void bwd_dq_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ Dsum, const float* __restrict__ Lse2,
    void* __restrict__ dQ, int Hq, int Hkv, int N_in, int npad, int BH, int nqb,
    float c /* scale * log2(e) */, float scale, const int* __restrict__ cu_seqlens, int window,
    const float* __restrict__ slopes, int out32) {
  constexpr int CH = D / 8, KK = D / 16, DB = D / 32;
  constexpr int NW = ROWS / 32;                     // waves per workgroup
  constexpr int TILE = kDqKeys * D;                 // 16-bit elements per tile
  constexpr int PIECES = TILE * 2 / 1024;           // 1 KB direct-load pieces per tile
  static_assert(PIECES % NW == 0, "each wave moves the same number of pieces");
  constexpr int PW = PIECES / NW;                   // pieces per wave per tile
  __shared__ __attribute__((aligned(1024))) short kv0[2 * TILE];
  __shared__ __attribute__((aligned(1024))) short kv1[2 * TILE];
  auto KV = [&](auto par) __attribute__((always_inline)) -> short* {
    if constexpr (decltype(par)::value == 0) return kv0; else return kv1;
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, g = lane >> 5, l32 = lane & 31;
  const int L = blockIdx.x;
  // block order as in the forward: heads in chunks of HC (32 when that divides B * Hq; packed
  // sequences: one sequence's heads), all query blocks of a chunk before the next, so that the
  // workgroups in flight share their heads' K/V tiles in L2
  const int HC = VARLEN ? Hq : ((BH % 32 == 0) ? 32 : BH);
  const int Lb = L % (HC * nqb);
  const int qblk = CAUSAL ? (nqb - 1 - Lb / HC) : (Lb / HC);
  const int bh = (L / (HC * nqb)) * HC + Lb % HC;
  const int h = bh % Hq, b = bh / Hq;
  const int kvh = h / (Hq / Hkv);
  const int bkv = b * Hkv + kvh;
  int N = N_in;
  size_t q_row0 = (size_t)bh * N_in;                // first row of the head in Q, dO, dQ
  size_t kv_off = (size_t)bkv * N_in * D;
  if constexpr (VARLEN) {
    const SeqRange sr = seq_range(cu_seqlens, b, N_in, npad);
    if (qblk * ROWS >= sr.n) return;                 // the whole workgroup: no barrier reached
    N = sr.n;
    q_row0 = (size_t)h * N_in + sr.s0;
    kv_off = ((size_t)kvh * N_in + sr.s0) * D;
  }
  const uint32_t head_bytes = (uint32_t)N * D * 2;
  const __amdgpu_buffer_rsrc_t qrs = make_rsrc(Q + q_row0 * D, head_bytes);
  const __amdgpu_buffer_rsrc_t ors = make_rsrc(dO + q_row0 * D, head_bytes);
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(K + kv_off, head_bytes);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(V + kv_off, head_bytes);

  const int q0 = qblk * ROWS;
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
  const float lse2 = qrow < N ? Lse2[(size_t)bh * npad + qrow] : INFINITY;
  const float dd = qrow < N ? Dsum[(size_t)bh * npad + qrow] : 0.f;
  // without a window or bias: -D of the lane's query in every register, the initial accumulator
  // of dP^T, so that the MFMAs deliver dP - D (the first MFMA of each chain reads it and none
  // overwrites it); the window / ALiBi variants, short of registers, add -D after the MFMAs
  f32x16_t ddv;
#pragma unroll
  for (int r = 0; r < 16; ++r) ddv[r] = EXT ? 0.f : dd;
  wait_all_loads();

  f32x16_t acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16_t{};

  // loop-invariant offsets.  Reads (16-bit units): K / V rows 32kb + l32 at chunk 2kk + g;
  // K^T through transposed reads of the K tile (tr_off).  Direct loads (bytes): piece NW i + w
  // of a tile, lane l -> LDS chunk 64(NW i + w) + l, fetched from the chunk the swizzle puts there.
  int off_row[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) off_row[kk] = chunk_index<D>(l32, 2 * kk + g) * 8;
  int off_tr[DB][2];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) off_tr[db][hh] = tr_off<D>(lane, db, hh);
  // piece NW i + w holds rows 64 NW i / CH further on than piece w, with the same swizzle (a
  // multiple of 16 rows), so its source is dma_kv + i * 64 NW / CH rows, a uniform offset
  static_assert((64 * NW / CH) % 16 == 0, "pieces of one wave keep the row swizzle");
  uint32_t dma_kv;
  {
    const int pch = 64 * w + lane;
    const int r = pch / CH, cc = pch % CH;
    dma_kv = ((uint32_t)r * D + ((cc ^ swz<D>(r)) << 3)) * 2;
  }
  auto load_tiles = [&](int j, auto par) __attribute__((always_inline)) {
    short* kv = KV(par);
    const uint32_t rowoff = (uint32_t)j * kDqKeys * D * 2;
#pragma unroll
    for (int i = 0; i < PW; ++i) {
      const int piece = NW * i + w;
      const uint32_t soff = rowoff + (uint32_t)i * (64 * NW / CH) * D * 2;
      buffer_load16_lds(krs, kv + 512 * piece, dma_kv, soff);
      buffer_load16_lds(vrs, kv + TILE + 512 * piece, dma_kv, soff);
    }
  };

  // window (0: none; capped at N, which already sees everything) and ALiBi slope in log2 units
  const int W = (EXT && window > 0) ? min(window, N) : 0;
  const float ab2 = ALIBI ? -slopes[h] * kLog2e : 0.f;
  const int kend = CAUSAL ? min(N, q0 + ROWS) : (W > 0 ? min(N, q0 + ROWS + W - 1) : N);
  const int ntiles = (kend + kDqKeys - 1) / kDqKeys;
  // first tile with a key inside the window of the block's first row
  const int jfirst = W > 0 ? max(0, q0 - W + 1) / kDqKeys : 0;
  // a wave takes part in tiles [jfirst, jact); under causal masking only tiles [jmask, jact)
  // cross its diagonal (EXT: every tile is masked)
  const int jact = (qw >= N) ? 0
                   : (CAUSAL ? min(ntiles, (qw + 31) / kDqKeys + 1)
                             : (W > 0 ? min(ntiles, (qw + 31 + W - 1) / kDqKeys + 1) : ntiles));
  const int jmask = EXT ? jfirst : (CAUSAL ? min(jact, q0 / kDqKeys) : jact);

  // S^T, dP^T for keys 32kb .. 32kb+31 of the tile in buffer `par`; lane owns query qrow,
  // register r holds key 32kb + 8(r/4) + 4g + r%4
  auto s_dp = [&](auto par, int kb, f32x16_t& st, f32x16_t& dpt) __attribute__((always_inline)) {
    const short* Kb = KV(par) + 32 * kb * D;
    const short* Vb = KV(par) + TILE + 32 * kb * D;
    st = f32x16_t{};
    dpt = ddv;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const i16x8_t ak = __builtin_bit_cast(i16x8_t, *(const uint4*)(Kb + off_row[kk]));
      const i16x8_t av = __builtin_bit_cast(i16x8_t, *(const uint4*)(Vb + off_row[kk]));
      st = mfma32x32x16<BF16>(ak, qf[kk], st);
      dpt = mfma32x32x16<BF16>(av, dof[kk], dpt);
    }
  };
  // dS^T = P^T (dP^T - D), packed as the B operand of dQ^T
  // mask_tag as in the dK/dV kernel: 0 none, 1 masked, 2 (EXT) bias only
  auto p_ds = [&](int kt0, int kb, f32x16_t& st, const f32x16_t& dpt, i16x8_t (&sb)[2],
                  auto mask_tag) __attribute__((always_inline)) {
    constexpr int MODE = (int)decltype(mask_tag)::value;
    constexpr bool MASK = MODE == 1;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float p;
      if constexpr (EXT && MODE != 0) {
        const int diff = qrow - (kt0 + 32 * kb + 8 * (r >> 2) + 4 * g + (r & 3));   // query - key
        float x = st[r] * c - lse2;
        if constexpr (ALIBI) x = __builtin_fmaf(__builtin_fabsf((float)diff), ab2, x);
        p = __builtin_amdgcn_exp2f(x);
        if constexpr (MASK) {
          const bool vis = (CAUSAL ? diff >= 0 : (W == 0 || diff > -W)) && (W == 0 || diff < W);
          if (!vis) p = 0.f;
        }
      } else if constexpr (EXT) {
        p = __builtin_amdgcn_exp2f(st[r] * c - lse2);
      } else {
        p = __builtin_amdgcn_exp2f(st[r] * c - lse2);
        if constexpr (MASK) {
          if (kt0 + 32 * kb + 8 * (r >> 2) + 4 * g + (r & 3) > qrow) p = 0.f;
        }
      }
      st[r] = EXT ? p * (dpt[r] + dd) : p * dpt[r];
    }
    sb[0] = pack8<BF16>(st, 0);
    sb[1] = pack8<BF16>(st, 8);
  };
  // dQ^T += K^T dS^T (slot (g, e) of half t is key 32kb + 16t + 8(e/4) + 4g + e%4)
  auto dq_mma = [&](auto par, int kb, const i16x8_t (&sb)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const i16x8_t a = read_tr8(KV(par) + (32 * kb + 16 * t) * D, off_tr[db]);
        acc[db] = mfma32x32x16<BF16>(a, sb[t], acc[db]);
      }
  };

  // One key tile j in buffer `par`: the S^T/dP^T MFMAs of the second 32 keys run beside the
  // dS work of the first, the dQ MFMAs of the first beside the dS work of the second.
  auto step = [&](int j, auto par, auto mask_tag) __attribute__((always_inline)) {
    using Other = std::integral_constant<int, 1 - decltype(par)::value>;
    if (j + 1 < ntiles) load_tiles(j + 1, Other{});
    const int kt0 = j * kDqKeys;
    f32x16_t s0, p0, s1, p1;
    i16x8_t sb0[2], sb1[2];
    s_dp(par, 0, s0, p0);
    p_ds(kt0, 0, s0, p0, sb0, mask_tag);
    s_dp(par, 1, s1, p1);
    p_ds(kt0, 1, s1, p1, sb1, mask_tag);
    dq_mma(par, 0, sb0);
    dq_mma(par, 1, sb1);
    // scheduling: LDS reads four ahead of their MFMAs (0x100 = LDS reads, 0x008 = MFMA,
    // 0x402 = vector ALU); the dQ MFMAs take two transposed reads each
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x402, 6, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
      __builtin_amdgcn_sched_group_barrier(0x402, 12, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
    }
    wait_all_loads();
    __syncthreads();
  };
  auto idle = [&](int j) __attribute__((always_inline)) {
    if (j + 1 < ntiles) {
      if (j & 1) load_tiles(j + 1, Par0{});
      else load_tiles(j + 1, Par1{});
    }
    wait_all_loads();
    __syncthreads();
  };

  if (jfirst & 1) load_tiles(jfirst, Par1{});
  else load_tiles(jfirst, Par0{});
  wait_all_loads();
  __syncthreads();
  int j = jfirst;
  auto run = [&](int end, auto mask_tag) __attribute__((always_inline)) {
    if ((j & 1) && j < end) {
      step(j, Par1{}, mask_tag);
      ++j;
    }
    for (; j + 1 < end; j += 2) {
      step(j, Par0{}, mask_tag);
      step(j + 1, Par1{}, mask_tag);
    }
    if (j < end) {
      step(j, Par0{}, mask_tag);
      ++j;
    }
  };
  if constexpr (EXT) {
    // tiles that cross a window edge or the diagonal for this wave's rows take the masked path,
    // tiles wholly inside the band the bias-only path with ALiBi, the plain path without (two
    // tile kinds per kernel)
    using Mode1 = std::integral_constant<int, 1>;
    using Inner = std::integral_constant<int, ALIBI ? 2 : 0>;
    for (; j < jact; ++j) {
      const int kt0 = j * kDqKeys;
      const int dmin = qw - (kt0 + kDqKeys - 1), dmax = qw + 31 - kt0;   // query - key
      const bool inside = (CAUSAL ? dmin >= 0 : (W == 0 || dmin > -W)) && (W == 0 || dmax < W);
      if (j & 1) {
        if (!inside) step(j, Par1{}, Mode1{});
        else step(j, Par1{}, Inner{});
      } else {
        if (!inside) step(j, Par0{}, Mode1{});
        else step(j, Par0{}, Inner{});
      }
    }
  } else {
    run(jmask, std::false_type{});
    for (; j < jact; ++j) {
      if (j & 1) step(j, Par1{}, std::true_type{});
      else step(j, Par0{}, std::true_type{});
    }
  }
  for (; j < ntiles; ++j) idle(j);

  // epilogue: dQ = scale * dQ^T; register r of block db holds d = 32db + 8(r/4) + 4g + r%4
  if (qrow < N) store_row<BF16, DB>(dQ, (q_row0 + qrow) * D, acc, scale, g, out32);
}

// ------------------------------------------------------------------ launchers
// Dense launches: N rows per head, workspace sized by N.  Variable-length launches (cu != nullptr):
// T packed rows per head in the tensors (passed as N), workspace and grid sized by max_seqlen.
template <bool BF16, int D, bool VARLEN>
static hipError_t launch_pre_t(const void* q, const void* k, const void* o, const void* dout, const float* lse, int B,
                               int Hq, int Hkv, int N, int max_seqlen, const int* cu, void* workspace,
                               hipStream_t stream) {
  (void)q;
  (void)k;
  (void)Hkv;
  const BwdWs w = bwd_ws(workspace, B, Hq, VARLEN ? max_seqlen : N);
  const unsigned grid = (unsigned)(B * Hq * (w.npad / kBwdRows));
  hipLaunchKernelGGL((bwd_pre_kernel<BF16, D, VARLEN>), dim3(grid), dim3(256), 0, stream, (const uint16_t*)o,
                     (const uint16_t*)dout, lse, w.dsum, w.lse2, N, w.npad, Hq, cu);
  return hipGetLastError();
}

template <bool BF16, int D, bool CAUSAL, bool VARLEN, bool EXT = false, bool ALIBI = false>
static hipError_t launch_dkdv_t(const void* q, const void* k, const void* v, const void* dout, const float* lse,
                                void* dk, void* dv, int B, int Hq, int Hkv, int N, int max_seqlen, const int* cu,
                                float scale, bool out32, const void* workspace, hipStream_t stream, int window = 0,
                                const float* slopes = nullptr) {
  (void)lse;   // the probabilities use LSE * log2(e) from the workspace
  const int rows = VARLEN ? max_seqlen : N;
  const BwdWs w = bwd_ws(const_cast<void*>(workspace), B, Hq, rows);
  const int nkb = (rows + kBwdKeys - 1) / kBwdKeys;
  const int ns = (VARLEN || EXT) ? 1 : dkdv_splits(B, Hq, Hkv, N);
  hipLaunchKernelGGL((bwd_dkdv_kernel<BF16, D, CAUSAL, VARLEN, EXT, ALIBI>), dim3(nkb * B * Hkv * ns), dim3(512), 0,
                     stream, (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)dout,
                     w.dsum, w.lse2, dk, dv, Hq, Hkv, N, w.npad, nkb, scale * kLog2e, scale, cu, window,
                     slopes, (int)out32, ns > 1 ? w.part : (float*)nullptr, ns);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || ns == 1) return e;
  const size_t n4 = (size_t)B * Hkv * N * D / 4;
  const unsigned grid = (unsigned)std::min<size_t>((2 * n4 + 255) / 256, 8192);
  hipLaunchKernelGGL((bwd_dkdv_sum_kernel<BF16>), dim3(grid), dim3(256), 0, stream, (const float*)w.part, dk, dv, n4,
                     ns, (int)out32);
  return hipGetLastError();
}

template <bool BF16, int D, bool CAUSAL, bool VARLEN, bool EXT = false, bool ALIBI = false>
static hipError_t launch_dq_t(const void* q, const void* k, const void* v, const void* dout, const float* lse,
                              void* dq, int B, int Hq, int Hkv, int N, int max_seqlen, const int* cu, float scale,
                              bool out32, const void* workspace, hipStream_t stream, int window = 0,
                              const float* slopes = nullptr) {
  (void)lse;
  const int rows = VARLEN ? max_seqlen : N;
  const BwdWs w = bwd_ws(const_cast<void*>(workspace), B, Hq, rows);
  const int BH = B * Hq;
  // 128-row blocks (4 waves) when 256-row blocks would give the CUs fewer than two workgroups
  // each, and at d = 128 for short rows (N <= 2048, or causal with N <= 4096), where the finer
  // blocks balance better (side by side: B=8 N=2048 causal 0.234 -> 0.218 ms, B=4 N=4096 causal
  // 0.391 -> 0.381, N=1024 causal 7% faster); plain dense layout only.  A row's arithmetic is the
  // same either way.
  if constexpr (!VARLEN && !EXT) {
    const bool short_rows = D == 128 && (rows <= 2048 || (CAUSAL && rows <= 4096));
    if ((long long)BH * ((rows + kDqRows - 1) / kDqRows) < 2 * kNumCUs || short_rows) {
      constexpr int R = kDqRows / 2;
      const int nqb = (rows + R - 1) / R;
      hipLaunchKernelGGL((bwd_dq_kernel<BF16, D, CAUSAL, VARLEN, EXT, R>), dim3(nqb * BH), dim3(R / 32 * 64), 0,
                         stream, (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)dout,
                         w.dsum, w.lse2, dq, Hq, Hkv, N, w.npad, BH, nqb, scale * kLog2e, scale, cu, window,
                         slopes, (int)out32);
      return hipGetLastError();
    }
  }
  const int nqb = (rows + kDqRows - 1) / kDqRows;
  hipLaunchKernelGGL((bwd_dq_kernel<BF16, D, CAUSAL, VARLEN, EXT, kDqRows, ALIBI>), dim3(nqb * BH),
                     dim3(kDqRows / 32 * 64), 0,
                     stream, (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)dout,
                     w.dsum, w.lse2, dq, Hq, Hkv, N, w.npad, BH, nqb, scale * kLog2e, scale, cu, window,
                     slopes, (int)out32);
  return hipGetLastError();
}

hipError_t launch_bwd_pre(const void* q, const void* k, const void* o, const void* dout, const float* lse, int B,
                          int Hq, int Hkv, int N, int d, bool bf16, void* workspace, hipStream_t stream,
                          int max_seqlen, const int* cu) {
  if (cu != nullptr) {
    if (bf16) return d == 128 ? launch_pre_t<true, 128, true>(q, k, o, dout, lse, B, Hq, Hkv, N, max_seqlen, cu, workspace, stream)
                              : launch_pre_t<true, 64, true>(q, k, o, dout, lse, B, Hq, Hkv, N, max_seqlen, cu, workspace, stream);
    return d == 128 ? launch_pre_t<false, 128, true>(q, k, o, dout, lse, B, Hq, Hkv, N, max_seqlen, cu, workspace, stream)
                    : launch_pre_t<false, 64, true>(q, k, o, dout, lse, B, Hq, Hkv, N, max_seqlen, cu, workspace, stream);
  }
  if (bf16) return d == 128 ? launch_pre_t<true, 128, false>(q, k, o, dout, lse, B, Hq, Hkv, N, N, cu, workspace, stream)
                            : launch_pre_t<true, 64, false>(q, k, o, dout, lse, B, Hq, Hkv, N, N, cu, workspace, stream);
  return d == 128 ? launch_pre_t<false, 128, false>(q, k, o, dout, lse, B, Hq, Hkv, N, N, cu, workspace, stream)
                  : launch_pre_t<false, 64, false>(q, k, o, dout, lse, B, Hq, Hkv, N, N, cu, workspace, stream);
}

#define EAO_DISPATCH_V(FN, VL, ...)                                                           \
  if (bf16) {                                                                                 \
    if (d == 128) {                                                                           \
      if (causal) return FN<true, 128, true, VL>(__VA_ARGS__);                                \
      return FN<true, 128, false, VL>(__VA_ARGS__);                                           \
    }                                                                                         \
    if (causal) return FN<true, 64, true, VL>(__VA_ARGS__);                                   \
    return FN<true, 64, false, VL>(__VA_ARGS__);                                              \
  }                                                                                           \
  if (d == 128) {                                                                             \
    if (causal) return FN<false, 128, true, VL>(__VA_ARGS__);                                 \
    return FN<false, 128, false, VL>(__VA_ARGS__);                                            \
  }                                                                                           \
  if (causal) return FN<false, 64, true, VL>(__VA_ARGS__);                                    \
  return FN<false, 64, false, VL>(__VA_ARGS__);

hipError_t launch_bwd_dkdv(const void* q, const void* k, const void* v, const void* dout, const float* lse, void* dk,
                           void* dv, int B, int Hq, int Hkv, int N, int d, bool causal, float scale, bool bf16,
                           bool out32, const void* workspace, hipStream_t stream, int max_seqlen, const int* cu) {
  if (cu != nullptr) {
    EAO_DISPATCH_V(launch_dkdv_t, true, q, k, v, dout, lse, dk, dv, B, Hq, Hkv, N, max_seqlen, cu, scale, out32,
                   workspace, stream)
  }
  EAO_DISPATCH_V(launch_dkdv_t, false, q, k, v, dout, lse, dk, dv, B, Hq, Hkv, N, N, cu, scale, out32, workspace,
                 stream)
}

hipError_t launch_bwd_dq(const void* q, const void* k, const void* v, const void* dout, const float* lse, void* dq,
                         int B, int Hq, int Hkv, int N, int d, bool causal, float scale, bool bf16, bool out32,
                         const void* workspace, hipStream_t stream, int max_seqlen, const int* cu) {
  if (cu != nullptr) {
    EAO_DISPATCH_V(launch_dq_t, true, q, k, v, dout, lse, dq, B, Hq, Hkv, N, max_seqlen, cu, scale, out32, workspace,
                   stream)
  }
  EAO_DISPATCH_V(launch_dq_t, false, q, k, v, dout, lse, dq, B, Hq, Hkv, N, N, cu, scale, out32, workspace, stream)
}
// sliding window and/or ALiBi (dense layout): the dK/dV and dQ phases with EXT
template <bool BF16, int D, bool CAUSAL, bool VARLEN, bool EXT_ = true>
static hipError_t launch_dkdv_ext_t(const void* q, const void* k, const void* v, const void* dout, const float* lse,
                                    void* dk, void* dv, int B, int Hq, int Hkv, int N, float scale, bool out32,
                                    const void* workspace, hipStream_t stream, int window, const float* slopes) {
  if (slopes != nullptr)
    return launch_dkdv_t<BF16, D, CAUSAL, false, true, true>(q, k, v, dout, lse, dk, dv, B, Hq, Hkv, N, N, nullptr,
                                                             scale, out32, workspace, stream, window, slopes);
  return launch_dkdv_t<BF16, D, CAUSAL, false, true, false>(q, k, v, dout, lse, dk, dv, B, Hq, Hkv, N, N, nullptr,
                                                            scale, out32, workspace, stream, window, slopes);
}
template <bool BF16, int D, bool CAUSAL, bool VARLEN, bool EXT_ = true>
static hipError_t launch_dq_ext_t(const void* q, const void* k, const void* v, const void* dout, const float* lse,
                                  void* dq, int B, int Hq, int Hkv, int N, float scale, bool out32,
                                  const void* workspace, hipStream_t stream, int window, const float* slopes) {
  if (slopes != nullptr)
    return launch_dq_t<BF16, D, CAUSAL, false, true, true>(q, k, v, dout, lse, dq, B, Hq, Hkv, N, N, nullptr, scale,
                                                           out32, workspace, stream, window, slopes);
  return launch_dq_t<BF16, D, CAUSAL, false, true, false>(q, k, v, dout, lse, dq, B, Hq, Hkv, N, N, nullptr, scale,
                                                          out32, workspace, stream, window, slopes);
}

hipError_t launch_bwd_dkdv_ext(const void* q, const void* k, const void* v, const void* dout, const float* lse,
                               void* dk, void* dv, int B, int Hq, int Hkv, int N, int d, bool causal, float scale,
                               bool bf16, bool out32, const void* workspace, hipStream_t stream, int window,
                               const float* slopes) {
  EAO_DISPATCH_V(launch_dkdv_ext_t, false, q, k, v, dout, lse, dk, dv, B, Hq, Hkv, N, scale, out32, workspace,
                 stream, window, slopes)
}

hipError_t launch_bwd_dq_ext(const void* q, const void* k, const void* v, const void* dout, const float* lse,
                             void* dq, int B, int Hq, int Hkv, int N, int d, bool causal, float scale, bool bf16,
                             bool out32, const void* workspace, hipStream_t stream, int window, const float* slopes) {
  EAO_DISPATCH_V(launch_dq_ext_t, false, q, k, v, dout, lse, dq, B, Hq, Hkv, N, scale, out32, workspace, stream,
                 window, slopes)
}
#undef EAO_DISPATCH_V

}  // namespace eao
