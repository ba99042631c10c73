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
//   * grid: one workgroup per (batch, query head, block of BR = NWV * QB * 32 query rows);
//     the NWV waves each own QB * 32 query rows.  The plain forward runs 8 waves (256 rows,
//     one workgroup and two waves per SIMD on a CU), so each K/V tile loaded into LDS serves
//     256 query rows, unless 256-row blocks would give the 256 CUs fewer than two workgroups
//     each (few batches x heads x rows): then 4 waves (128 rows, twice the workgroups), which
//     fills the idle CUs; each row's arithmetic is the same either way.  The variants with
//     window/ALiBi (more registers) and variable lengths (finer early exit) run 4.  The heads are taken in chunks (32 heads, or one packed
//     sequence's heads) so that the workgroups in flight share K/V tiles in L2; within a chunk,
//     causal launches visit the longest query blocks first, so short blocks fill the tail.
//   * transposed formulation: each wave computes S^T = K Q^T and O^T = V^T P^T with
//     v_mfma_f32_32x32x16.  In the S^T accumulator a lane owns one query (column l % 32) and 16
//     keys, so the row maximum and row sum are lane-local; one v_permlane32_swap combines the
//     two lane halves.  O^T's accumulator has the same lane -> query ownership, so the rescale
//     by exp(m_old - m_new) is one multiply per register, and the S^T accumulator, converted
//     to 16-bit, is directly the B operand (P^T) of the second MFMA (k relabelled, see
//     common.hpp).
//   * Q stays in registers for the whole key loop (B operand of S^T).  K and V tiles of BC keys
//     go straight from HBM into double-buffered, XOR-swizzled LDS tiles with direct
//     buffer -> LDS loads (no staging registers); K is read with ds_read_b128 and V through
//     ds_read_b64_tr_b16, which delivers V^T fragments without a separate transpose.
//   * software pipeline: K runs one tile ahead of V, so while the softmax of tile j runs on the
//     vector ALU, the MFMAs of S^T for tile j + 1 are already issued; both sit in one basic block
//     and the scheduler interleaves them (a single wave keeps the matrix core and the vector
//     ALU busy together).
//   * softmax in base 2: the running maximum is kept in units of s * scale * log2(e), so each
//     probability is one fma plus one v_exp_f32.
#include <type_traits>

#include "common.hpp"

namespace eao {

// Headroom (log2 units) of the deferred rescaling: probabilities stay <= 2^kStaleMax.
constexpr float kStaleMax = 8.0f;
// Running maximum of a row that has seen no visible key yet: finite and below any score, so the
// first visible key always takes the rescale branch (its factor 2^(kMUnset - m) is 0) and the
// exponentials need no test for an unset maximum (2^(-inf - kMUnset) = 0 for masked keys).
constexpr float kMUnset = -1e30f;

// LDS tiles (K and V, [BC keys][D], double-buffered each) are unpadded, with 16-byte chunks
// XOR-swizzled by row (swz in common.hpp): a ds_read_b128 of 16 consecutive rows at one
// chunk, and a ds_read_b64_tr_b16 of 4 consecutive rows x 4 consecutive chunks, both hit
// distinct bank groups.  Unpadded rows let the tiles be filled by direct buffer -> LDS loads
// (each instruction moves 64 lanes x 16 bytes to 1 KB of consecutive LDS; the swizzle is
// applied by choosing which global chunk each lane fetches), so staging takes no registers.
template <int D, int BC>
struct FwdTile {
  static constexpr int CH = D / 8;                 // 16-byte chunks per row
  static constexpr int ELEMS = BC * D;             // 16-bit elements per tile
  static constexpr int PIECES = ELEMS * 2 / 1024;  // 1 KB direct-load pieces per tile
};


// EXT adds the local (sliding-window) mask and the ALiBi bias ("FlashAttention-2: Faster Attention
// with Better Parallelism and Work Partitioning", OpenReview discussion, author responses: FA2
// supports ALiBi and local, i.e. sliding-window, attention): with window > 0, key j is visible to
// query i only if i - j < window (and, without the causal mask, j - i < window); with slopes,
// score (i, j) of head h gets - slopes[h] * |i - j| added after the softmax scale.  Every tile
// of an EXT launch takes the masked path; tiles wholly before the window start of the
// workgroup's first row are not visited.
//
// VARLEN: sequences of different lengths packed without padding ("FlashAttention-2: Faster
// Attention with Better Parallelism and Work Partitioning", OpenReview discussion, author
// responses: variable sequence lengths, concatenated with an array of lengths).  Q, K, V, O are
// [H, T, d] and LSE [H, T] with T = N_in packed tokens; sequence b is rows cu_seqlens[b] ..
// cu_seqlens[b + 1] - 1 of every head (clamped to [0, T]) and attends only within itself.  The
// grid covers the longest sequence (nqb blocks of BR rows); blocks past a sequence's end exit.
template <bool BF16, int D, int QB, int BC, bool CAUSAL, bool EXT = false, bool VARLEN = false, int NWV = 4,
          bool ALIBI = false>
__global__ __launch_bounds__(NWV * 64, (EXT || NWV == 8) ? 1 : 2) void attn_fwd_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    uint16_t* __restrict__ O, float* __restrict__ LSE, int Hq, int Hkv, int N_in, int BH, int nqb,
    float c /* softmax_scale * log2(e) */, int window, const float* __restrict__ slopes, float inv_scale,
    const int* __restrict__ cu_seqlens) {
  using T = FwdTile<D, BC>;
  constexpr int CH = T::CH, KK = D / 16, DB = D / 32, KB = BC / 32;
  constexpr int BR = NWV * QB * 32;
  static_assert(T::PIECES % NWV == 0, "each wave moves the same number of pieces");
  // four distinct LDS objects, so that the compiler can tell a direct load into one buffer from
  // a read of another and does not wait for the load before the read
  __shared__ __attribute__((aligned(1024))) short k_lds0[T::ELEMS];
  __shared__ __attribute__((aligned(1024))) short k_lds1[T::ELEMS];
  __shared__ __attribute__((aligned(1024))) short v_lds0[T::ELEMS];
  __shared__ __attribute__((aligned(1024))) short v_lds1[T::ELEMS];
  auto Ks = [&](auto par) -> short* __attribute__((always_inline)) {
    if constexpr (decltype(par)::value == 0) return k_lds0; else return k_lds1;
  };
  auto Vs = [&](auto par) -> short* __attribute__((always_inline)) {
    if constexpr (decltype(par)::value == 0) return v_lds0; else return v_lds1;
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, g = lane >> 5, l32 = lane & 31;
  const int G16 = lane >> 4, li = lane & 15;
  const int L = blockIdx.x;
  // Block order: the heads are taken in chunks of HC (32 when that divides B * Hq; packed
  // sequences: one sequence's heads), all query blocks of a chunk before the next chunk, block
  // by block across the chunk's heads (causal: longest blocks first).  The workgroups in flight
  // then share their heads' K/V tiles in L2 instead of spreading over every head.
  const int HC = VARLEN ? Hq : ((BH % 32 == 0) ? 32 : BH);
  const int Lb = L % (HC * nqb);
  const int qblk = CAUSAL ? (nqb - 1 - Lb / HC) : (Lb / HC);
  const int bh = (L / (HC * nqb)) * HC + Lb % HC;
  const int h = bh % Hq, b = bh / Hq;
  const int kvh = h / (Hq / Hkv);
  int N = N_in;
  size_t q_off, kv_off, lse_off;
  if constexpr (VARLEN) {
    const int s0 = min(max(cu_seqlens[b], 0), N_in);
    const int s1 = min(max(cu_seqlens[b + 1], s0), N_in);
    N = s1 - s0;
    if (qblk * BR >= N) return;               // the whole workgroup: no barrier has been reached
    q_off = ((size_t)h * N_in + s0) * D;
    kv_off = ((size_t)kvh * N_in + s0) * D;
    lse_off = (size_t)h * N_in + s0;
  } else {
    q_off = ((size_t)b * Hq + h) * (size_t)N * D;
    kv_off = ((size_t)b * Hkv + kvh) * (size_t)N * D;
    lse_off = (size_t)bh * N;
  }
  const uint16_t* Qp = Q + q_off;

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
    m[qb] = kMUnset;
    l[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) o[qb][db] = f32x16_t{};
  }

  const bool win = EXT && window > 0;
  const int kend = CAUSAL ? min(N, q0 + BR) : (win ? min(N, q0 + BR - 1 + window) : N);
  const int ntiles = (kend + BC - 1) / BC;
  // first tile with a key inside the window of the workgroup's first row
  const int jfirst = win ? max(0, q0 - window + 1) / BC : 0;
  // ALiBi in units of the raw scores (the softmax scale multiplies later): -slope / scale
  const float ab = ALIBI ? -slopes[h] * inv_scale : 0.f;

  // K/V of this head through bounds-checked buffer loads: keys >= N read as zeros
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(K + kv_off, (uint32_t)N * D * 2);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(V + kv_off, (uint32_t)N * D * 2);
  // direct loads: piece p = NWV i + w of a tile; lane l fills LDS chunk 64p + l (row (64p + l) / CH,
  // physical chunk l % CH) with the logical chunk that the swizzle puts there
  // (piece NWV i + w lies 64 NWV i / CH rows after piece w, a multiple of the swizzle's period,
  // so its source is goff plus a uniform offset)
  static_assert((64 * NWV / CH) % 16 == 0, "pieces of one wave keep the row swizzle");
  uint32_t goff;
  {
    const int p = 64 * w + lane;
    const int row = p / CH, pch = p % CH;
    goff = ((uint32_t)row * D + ((pch ^ swz<D>(row)) << 3)) * 2;
  }
  auto load_tile = [&](__amdgpu_buffer_rsrc_t rs, short* dst, int kt0) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < T::PIECES / NWV; ++i)
      buffer_load16_lds(rs, dst + 512 * (NWV * i + w), goff,
                        (uint32_t)kt0 * D * 2 + (uint32_t)i * (64 * NWV / CH) * D * 2);
  };

  // loop-invariant LDS offsets (16-bit units): K rows l32 (+32 kb) at chunk 2kk + g; V^T
  // transposed reads at rows 4(G16/2) + li/4 (+8h, +16t, +32kb), columns 32db + 16(G16%2) + 4(li%4)
  int off_k[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) off_k[kk] = chunk_index<D>(l32, 2 * kk + g) * 8;
  int off_v[DB][2];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
      off_v[db][hh] = elem_index<D>(4 * (G16 >> 1) + (li >> 2) + 8 * hh, 32 * db + 16 * (G16 & 1) + 4 * (li & 3));

  // a wave takes part in tiles [0, jact): under causal masking, tiles whose first key lies after
  // the wave's last query row are skipped (the wave still helps stage them)
  const int jact = (qw >= N) ? 0
                   : (CAUSAL ? min(ntiles, qw_last / BC + 1)
                             : (win ? min(ntiles, (qw_last + window - 1) / BC + 1) : ntiles));

  // S^T = K Q^T for the key tile in K buffer `par`
  auto compute_s = [&](auto par, f32x16_t (&s)[QB][KB]) __attribute__((always_inline)) {
    const short* Kb = Ks(par);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) s[qb][kb] = f32x16_t{};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const i16x8_t a = __builtin_bit_cast(i16x8_t, *(const uint4*)(Kb + 32 * kb * D + off_k[kk]));
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[qb][kb] = mfma32x32x16<BF16>(a, qf[qb][kk], s[qb][kb]);
      }
    }
  };

  // staging of one iteration: K_{j+2} replaces K_j (read while computing S^T of tile j, one
  // iteration ago), V_{j+1} replaces V_{j-1} (read one iteration ago)
  // (tile j lives in K and V buffers j % 2 = par)
  auto stage = [&](int j, auto par) __attribute__((always_inline)) {
    using Other = std::integral_constant<int, 1 - decltype(par)::value>;
    if (j + 2 < ntiles) load_tile(krs, Ks(par), (j + 2) * BC);
    if (j + 1 < ntiles) load_tile(vrs, Vs(Other{}), (j + 1) * BC);
  };
  // the loads of this iteration have landed in LDS and every wave is done with this tile
  auto publish = [&]() __attribute__((always_inline)) {
    wait_all_loads();
    __syncthreads();
  };

  // One key tile j, software-pipelined: S^T of tile j is already in sc (computed one iteration
  // earlier).  After the row maxima and the (rare) rescale, one basic block holds the MFMAs of
  // S^T for tile j + 1 (into sn), the exponentials of tile j and its O^T += V^T P^T, so the
  // scheduler overlaps matrix and vector work.  MASK selects the variant with causal / key-tail
  // masking.
  f32x16_t sA[QB][KB], sB[QB][KB];   // S^T of even / odd tiles
  // MODE 0: no mask; 1: masked (causal diagonal, key tail, window edges; with ALIBI also the
  // bias); 2: no mask, ALiBi bias only (ALIBI tiles inside the band)
  auto body = [&](int j, auto par, auto mode_tag) __attribute__((always_inline)) {
    constexpr int MODE = decltype(mode_tag)::value;
    constexpr bool MASK = MODE == 1;
    constexpr int P = decltype(par)::value;
    using Other = std::integral_constant<int, 1 - P>;
    auto& sc = P == 0 ? sA : sB;
    auto& sn = P == 0 ? sB : sA;
    const int kt0 = j * BC;
    stage(j, par);
    // ---- row maxima of tile j; rescale when a row's maximum has grown by more than kStaleMax
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      if constexpr (EXT && MODE != 0) {
        // distance qrow - key of register r as an exact float: (qrow - kt0 - 4g) - constant
        const int qrow = qw + 32 * qb + l32;
        const float dq = (float)(qrow - kt0 - 4 * g);
        const float lo = (float)(qrow - N);                 // key >= N  <=>  qrow - key <= lo
        const float wf = win ? (float)window : INFINITY;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float diff = dq - (float)(32 * kb + 8 * (r >> 2) + (r & 3));
            float val = sc[qb][kb][r];
            if constexpr (ALIBI) val = __builtin_fmaf(__builtin_fabsf(diff), ab, val);
            if constexpr (MASK) {
              const bool vis = diff > lo && diff < wf && (CAUSAL ? diff >= 0.f : diff > -wf);
              val = vis ? val : -INFINITY;
            }
            sc[qb][kb][r] = val;
          }
      } else if constexpr (MASK) {
        const int qrow = qw + 32 * qb + l32;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kt0 + 32 * kb + 8 * (r >> 2) + 4 * g + (r & 3);
            if (key >= N || (CAUSAL && key > qrow)) sc[qb][kb][r] = -INFINITY;
          }
      }
      const float mt = row_max(sc[qb]) * c;
      // The accumulator is rescaled only when some row's maximum has grown by more than
      // kStaleMax (log2 units) since the last rescale; otherwise the stale maximum is kept,
      // probabilities stay <= 2^kStaleMax, and the final division by l (computed against the
      // same maximum) gives the same result.  The decision is per row (alpha is exactly 1
      // where the row keeps its maximum), so a row's result never depends on other rows; the
      // branch only skips the multiplies when no row of the wave needs them.
      const bool grow = mt > m[qb] + kStaleMax;
      if (__builtin_amdgcn_ballot_w64(grow) != 0) {
        float alpha = grow ? __builtin_amdgcn_exp2f(m[qb] - mt) : 1.f;
        // an opaque (volatile) definition of alpha pins the multiplies inside this branch
        asm volatile("" : "+v"(alpha));
        m[qb] = grow ? mt : m[qb];
        l[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) o[qb][db] *= alpha;
      }
    }
    // ---- S^T of the next tile (past the wave's last tile it reads a stale buffer and the
    // result is never used), probabilities of tile j, O^T += V^T P^T
    compute_s(Other{}, sn);
    i16x8_t pf[QB][KB][2];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float rs4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = __builtin_amdgcn_exp2f(sc[qb][kb][r] * c - m[qb]);
          sc[qb][kb][r] = p;
          rs4[r & 3] += p;
        }
      l[qb] += (rs4[0] + rs4[1]) + (rs4[2] + rs4[3]);
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        pf[qb][kb][0] = pack8<BF16>(sc[qb][kb], 0);
        pf[qb][kb][1] = pack8<BF16>(sc[qb][kb], 8);
      }
    }
    const short* Vb = Vs(par);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int rb = (32 * kb + 16 * t) * D;   // 16 | row offset keeps the swizzle unchanged
          const i16x4_t lo = ds_read_tr16(Vb + rb + off_v[db][0]);
          const i16x4_t hi = ds_read_tr16(Vb + rb + off_v[db][1]);
          const i16x8_t a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) o[qb][db] = mfma32x32x16<BF16>(a, pf[qb][kb][t], o[qb][db]);
        }
    publish();
  };
  // staging only, for tiles this wave skips
  auto idle = [&](int j) __attribute__((always_inline)) {
    if (j & 1) stage(j, Par1{});
    else stage(j, Par0{});
    publish();
  };

  // prologue: K and V of tile jfirst, K of tile jfirst + 1 staged; S^T of tile jfirst (tile j
  // lives in the buffers of parity j % 2; jfirst is 0 unless a window skips leading tiles)
  auto prologue = [&](auto par) __attribute__((always_inline)) {
    using Other = std::integral_constant<int, 1 - decltype(par)::value>;
    load_tile(krs, Ks(par), jfirst * BC);
    load_tile(vrs, Vs(par), jfirst * BC);
    if (jfirst + 1 < ntiles) load_tile(krs, Ks(Other{}), (jfirst + 1) * BC);
    publish();
    if (jact > jfirst) compute_s(par, decltype(par)::value == 0 ? sA : sB);
  };
  if (jfirst & 1) prologue(Par1{});
  else prologue(Par0{});
  // the first iteration overwrites the K buffer of tile jfirst
  __syncthreads();

  // tiles [jlo, jmask) need no masking for any wave of the workgroup: below the causal diagonal
  // (keys < q0), before the key tail, and (window) inside the band of every row of the block;
  // tiles [jfirst, jlo) and [jmask, jact) are masked
  using Mode0 = std::integral_constant<int, 0>;
  using Mode1 = std::integral_constant<int, 1>;
  using Mode2 = std::integral_constant<int, 2>;
  int jmask = min(jact, CAUSAL ? min(q0, N) / BC : N / BC);
  int jlo = jfirst;
  if (win) {
    jlo = max(jfirst, (max(0, q0 + BR - window) + BC - 1) / BC);
    if (!CAUSAL) jmask = min(jmask, (q0 + window) / BC);
  }
  jmask = max(jmask, jlo);
  int j = jfirst;
  auto run_masked = [&](int end) __attribute__((always_inline)) {
    for (; j < end; ++j) {
      if (j & 1) body(j, Par1{}, Mode1{});
      else body(j, Par0{}, Mode1{});
    }
  };
  if constexpr (EXT) {
    // the tile's kind chosen per tile, two kinds per instantiation (masked, and bias-only with
    // ALIBI or plain without); the loop runs over pairs of tiles so that the buffer parity (and
    // with it which S^T registers hold the current and the next tile) is fixed at compile time
    // in each half
    using Inner = std::integral_constant<int, ALIBI ? 2 : 0>;
    auto ext_body = [&](int jj, auto par) __attribute__((always_inline)) {
      if (jj >= jlo && jj < jmask) body(jj, par, Inner{});
      else body(jj, par, Mode1{});
    };
    if ((j & 1) && j < jact) {
      ext_body(j, Par1{});
      ++j;
    }
    for (; j + 2 <= jact; j += 2) {
      ext_body(j, Par0{});
      ext_body(j + 1, Par1{});
    }
    if (j < jact) {
      ext_body(j, Par0{});
      ++j;
    }
  } else {
    // jfirst = jlo = 0: tiles [0, jmask) in pairs of parities 0, 1
    for (; j + 2 <= jmask; j += 2) {
      body(j, Par0{}, Mode0{});
      body(j + 1, Par1{}, Mode0{});
    }
    if (j < jmask) {
      body(j, Par0{}, Mode0{});
      ++j;
    }
  }
  run_masked(jact);
  for (; j < ntiles; ++j) idle(j);

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
      if (g == 0) LSE[lse_off + qrow] = (m[qb] + __log2f(lt)) * kLn2;
    }
  }
}

template <bool BF16, int D, int QB, int BC, bool CAUSAL, int NWV>
static hipError_t launch_fwd_nwv(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
                                 int Hkv, int N, float scale, hipStream_t stream) {
  constexpr int BR = NWV * QB * 32;
  const int nqb = (N + BR - 1) / BR;
  const int BH = B * Hq;
  auto kern = attn_fwd_kernel<BF16, D, QB, BC, CAUSAL, false, false, NWV>;
  hipLaunchKernelGGL(kern, dim3(nqb * BH), dim3(NWV * 64), 0, stream, (const uint16_t*)q, (const uint16_t*)k,
                     (const uint16_t*)v, (uint16_t*)o, lse, Hq, Hkv, N, BH, nqb, scale * kLog2e, 0,
                     (const float*)nullptr, 1.f, (const int*)nullptr);
  return hipGetLastError();
}

// 256-row blocks when they give every CU at least two workgroups, else 128-row blocks
template <bool BF16, int D, int QB, int BC, bool CAUSAL>
static hipError_t launch_fwd_t(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
                               int Hkv, int N, float scale, hipStream_t stream) {
  const long long blocks8 = (long long)B * Hq * ((N + 8 * QB * 32 - 1) / (8 * QB * 32));
  if (blocks8 < 2 * kNumCUs)
    return launch_fwd_nwv<BF16, D, QB, BC, CAUSAL, 4>(q, k, v, o, lse, B, Hq, Hkv, N, scale, stream);
  return launch_fwd_nwv<BF16, D, QB, BC, CAUSAL, 8>(q, k, v, o, lse, B, Hq, Hkv, N, scale, stream);
}

template <bool BF16, int D, bool CAUSAL, int NWV, bool ALIBI>
static hipError_t launch_fwd_ext_w(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
                                   int Hkv, int N, float scale, int window, const float* slopes, hipStream_t stream) {
  constexpr int BR = NWV * 32;
  const int nqb = (N + BR - 1) / BR;
  const int BH = B * Hq;
  hipLaunchKernelGGL((attn_fwd_kernel<BF16, D, 1, 64, CAUSAL, true, false, NWV, ALIBI>), dim3(nqb * BH),
                     dim3(NWV * 64), 0, stream, (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v,
                     (uint16_t*)o, lse, Hq, Hkv, N, BH, nqb, scale * kLog2e, window, slopes, 1.f / scale,
                     (const int*)nullptr);
  return hipGetLastError();
}

// window / ALiBi: ALiBi is a compile-time switch (each kernel then has two tile kinds); 256-row
// blocks when they give every CU at least two workgroups, else 128-row blocks
template <bool BF16, int D, bool CAUSAL>
static hipError_t launch_fwd_ext_t(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
                                   int Hkv, int N, float scale, int window, const float* slopes, hipStream_t stream) {
  const bool big = (long long)B * Hq * ((N + 255) / 256) >= 2 * kNumCUs;
  if (slopes != nullptr) {
    if (big) return launch_fwd_ext_w<BF16, D, CAUSAL, 8, true>(q, k, v, o, lse, B, Hq, Hkv, N, scale, window, slopes, stream);
    return launch_fwd_ext_w<BF16, D, CAUSAL, 4, true>(q, k, v, o, lse, B, Hq, Hkv, N, scale, window, slopes, stream);
  }
  if (big) return launch_fwd_ext_w<BF16, D, CAUSAL, 8, false>(q, k, v, o, lse, B, Hq, Hkv, N, scale, window, slopes, stream);
  return launch_fwd_ext_w<BF16, D, CAUSAL, 4, false>(q, k, v, o, lse, B, Hq, Hkv, N, scale, window, slopes, stream);
}

hipError_t launch_fwd_ext(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv,
                          int N, int d, bool causal, float scale, bool bf16, int window, const float* slopes,
                          hipStream_t stream) {
#define EAO_FWDX(BF, DD, CA) \
  return launch_fwd_ext_t<BF, DD, CA>(q, k, v, o, lse, B, Hq, Hkv, N, scale, window, slopes, stream)
  if (bf16) {
    if (d == 128) { if (causal) EAO_FWDX(true, 128, true); else EAO_FWDX(true, 128, false); }
    else { if (causal) EAO_FWDX(true, 64, true); else EAO_FWDX(true, 64, false); }
  } else {
    if (d == 128) { if (causal) EAO_FWDX(false, 128, true); else EAO_FWDX(false, 128, false); }
    else { if (causal) EAO_FWDX(false, 64, true); else EAO_FWDX(false, 64, false); }
  }
#undef EAO_FWDX
}

template <bool BF16, int D, bool CAUSAL>
static hipError_t launch_fwd_varlen_t(const void* q, const void* k, const void* v, void* o, float* lse,
                                      const int* cu_seqlens, int B, int Hq, int Hkv, int T, int max_seqlen,
                                      float scale, hipStream_t stream) {
  constexpr int BR = 128;
  const int nqb = (max_seqlen + BR - 1) / BR;
  const int BH = B * Hq;
  hipLaunchKernelGGL((attn_fwd_kernel<BF16, D, 1, 64, CAUSAL, false, true>), dim3(nqb * BH), dim3(256), 0, stream,
                     (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (uint16_t*)o, lse, Hq, Hkv, T, BH,
                     nqb, scale * kLog2e, 0, (const float*)nullptr, 1.f, cu_seqlens);
  return hipGetLastError();
}

hipError_t launch_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse, const int* cu_seqlens,
                             int B, int Hq, int Hkv, int T, int max_seqlen, int d, bool causal, float scale,
                             bool bf16, hipStream_t stream) {
#define EAO_FWDV(BF, DD, CA) \
  return launch_fwd_varlen_t<BF, DD, CA>(q, k, v, o, lse, cu_seqlens, B, Hq, Hkv, T, max_seqlen, scale, stream)
  if (bf16) {
    if (d == 128) { if (causal) EAO_FWDV(true, 128, true); else EAO_FWDV(true, 128, false); }
    else { if (causal) EAO_FWDV(true, 64, true); else EAO_FWDV(true, 64, false); }
  } else {
    if (d == 128) { if (causal) EAO_FWDV(false, 128, true); else EAO_FWDV(false, 128, false); }
    else { if (causal) EAO_FWDV(false, 64, true); else EAO_FWDV(false, 64, false); }
  }
#undef EAO_FWDV
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
