// Split-KV forward for decoding: few query rows per head against a long key/value sequence.
//
// Method ("FlashAttention-2: Faster Attention with Better Parallelism and Work Partitioning",
// OpenReview discussion: the author response on decoding, where the original kernel lacked
// parallelism over long keys, and the review summary, where the KV cache is split among thread
// blocks to saturate memory bandwidth; the merge uses the saved logsumexp of each part): the
// keys of one (batch, K/V head) are cut into S contiguous splits, each split computes the exact
// softmax-weighted partial result of its keys with the online softmax and its logsumexp, and a
// second kernel combines the parts exactly:
//   LSE = ln sum_s exp(LSE_s),  O = sum_s exp(LSE_s - LSE) O_s.
//
// gfx950 mapping
//   * split kernel: one workgroup of one wave per (batch, K/V head, split, group of 32 rows).
//     The query rows that use the K/V head -- G = Hq / Hkv heads times Nq rows -- are taken 32 at
//     a time as the 32 columns of one MFMA tile (transposed formulation as in the main forward:
//     a lane owns one row); the workgroups of one split's row groups are adjacent in the grid,
//     so beyond the first they find the split's keys in L2.  The wave streams its split's keys
//     in stages of 32 (one MFMA tile of keys) through a ring of four LDS slots filled by direct
//     buffer -> LDS loads issued three stages ahead, and waits only for the oldest stage (a
//     counter wait; the wave is alone in its workgroup, so there is no barrier): two to three
//     stages, 32-48 KB at d = 128, stay in flight per wave.  The kernel is bound by HBM
//     bandwidth (every key is read once per K/V head); a double-buffered tile shared by four
//     waves left at most one tile in flight, which drained before each new request.
//   * merge kernel: one wave per output row.
//
// Causal alignment for Nq < Nk (bottom-right): query i sits at position Nk - Nq + i and sees
// keys j <= Nk - Nq + i.
#include <atomic>
#include <mutex>

#include "common.hpp"

namespace eao {

constexpr int kSkTile = 128;   // split granularity: every split but the last holds a multiple of 128 keys
constexpr int kSkStage = 32;   // keys per pipeline stage
constexpr int kSkSlots = 4;    // LDS ring slots (stages) per wave

// Wait until at most n of this wave's vector-memory operations are outstanding and its LDS
// operations have completed (vmcnt is six bits on gfx9: bits 3:0 and 15:14; expcnt left at 7).
template <int n>
__device__ __forceinline__ void wait_vmem_lds() {
  static_assert(n >= 0 && n < 64, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(0x0070 | (n & 15) | ((n >> 4) << 14));
}

// Static scratch of the allocation-free entry point: the split partials (float O and LSE of
// every split) live here instead of in a caller's workspace.  Each GPU holds its own copy for
// the life of the process.  In host code `scratch` only names the symbol; its device address
// comes from hipGetSymbolAddress (splitkv_scratch_address below) and is the only form passed to
// kernels.
constexpr size_t kSplitkvScratchBytes = (size_t)8 << 20;
static __device__ __attribute__((aligned(256))) unsigned char scratch[kSplitkvScratchBytes];

size_t splitkv_scratch_bytes() { return kSplitkvScratchBytes; }

// Device address of `scratch` on the current device: looked up once per device (with that
// device current, as the entry point runs) and kept.
hipError_t splitkv_scratch_address(void** out) {
  constexpr int kMaxDevices = 64;
  static std::atomic<void*> addr[kMaxDevices];
  static std::mutex init_mu;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(init_mu);
    p = addr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (p == nullptr) return hipErrorInvalidSymbol;
      addr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}

// groups of 32 query rows per K/V head
static int splitkv_row_groups(int Hq, int Hkv, int Nq) { return ((Hq / Hkv) * Nq + 31) / 32; }

// keys per split (a multiple of the tile) and number of splits for a launch
void splitkv_plan(int B, int Hq, int Hkv, int Nq, int Nk, int num_splits, int* splits, int* keys_per_split) {
  const int tiles = (Nk + kSkTile - 1) / kSkTile;
  int s = num_splits;
  if (s <= 0) {
    // about two workgroups (waves) per compute unit -- as many as the LDS of one CU holds at
    // d = 128 -- but splits of at least 4 x 128 keys: shorter splits spend more time in their
    // first load and the merge than they save
    const int wg = B * Hkv * splitkv_row_groups(Hq, Hkv, Nq);
    const int want = (2 * 256 + wg - 1) / wg;
    s = want < tiles / 4 ? want : tiles / 4;
  }
  s = s < 1 ? 1 : (s > tiles ? tiles : s);
  const int tps = (tiles + s - 1) / s;                     // tiles per split
  *keys_per_split = tps * kSkTile;
  *splits = (tiles + tps - 1) / tps;                        // no empty split
}

size_t splitkv_workspace_bytes(int B, int Hq, int Hkv, int Nq, int Nk, int d, int num_splits) {
  int s, l;
  splitkv_plan(B, Hq, Hkv, Nq, Nk, num_splits, &s, &l);
  const size_t rows = (size_t)s * B * Hq * Nq;
  return (rows * d * 4 + 255) / 256 * 256 + (rows * 4 + 255) / 256 * 256;
}

template <bool BF16, int D, bool CAUSAL>
__global__ __launch_bounds__(64) void fwd_split_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                                                      const uint16_t* __restrict__ V, float* __restrict__ Opart,
                                                      float* __restrict__ Lpart, int B, int Hq, int Hkv, int Nq, int Nk,
                                                      int S, int L, float c /* scale * log2(e) */) {
  constexpr int CH = D / 8, KK = D / 16, DB = D / 32;
  constexpr int STAGE = kSkStage * D;               // 16-bit elements of K (or V) per stage
  constexpr int PIECES = STAGE * 2 / 1024;          // 1 KB direct loads per tensor and stage
  constexpr int LPS = 2 * PIECES;                   // loads per stage (K and V)
  static_assert(PIECES * 64 * 8 == STAGE, "a stage is whole 1 KB pieces");
  static_assert(2 * LPS < 64, "two stages' loads fit the counter");
  // four slots [K | V], distinct objects so that the compiler tracks each slot's loads apart
  __shared__ __attribute__((aligned(1024))) short kv0[2 * STAGE];
  __shared__ __attribute__((aligned(1024))) short kv1[2 * STAGE];
  __shared__ __attribute__((aligned(1024))) short kv2[2 * STAGE];
  __shared__ __attribute__((aligned(1024))) short kv3[2 * STAGE];
  auto slot = [&](auto sl) __attribute__((always_inline)) -> short* {
    constexpr int SL = decltype(sl)::value;
    if constexpr (SL == 0) return kv0;
    else if constexpr (SL == 1) return kv1;
    else if constexpr (SL == 2) return kv2;
    else return kv3;
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;
  using S3 = std::integral_constant<int, 3>;

  const int lane = threadIdx.x;
  const int g = lane >> 5, l32 = lane & 31;
  const int G = Hq / Hkv, R = G * Nq, RG = (R + 31) / 32;
  const int rg = blockIdx.x % RG, s = (blockIdx.x / RG) % S, bkv = blockIdx.x / (RG * S);
  const int b = bkv / Hkv, kvh = bkv % Hkv;
  // this lane's query row: head kvh * G + row / Nq, row row % Nq (rows >= R are padding)
  const int row = 32 * rg + l32;
  const bool row_ok = row < R;
  const int gh = row_ok ? row / Nq : 0, qi = row_ok ? row % Nq : 0;
  const int hq = kvh * G + gh;
  const int qpos = Nk - Nq + qi;                    // the row's position among the keys

  i16x8_t qf[KK];
  {
    const uint16_t* qp = Q + (((size_t)b * Hq + hq) * Nq + qi) * D;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      qf[kk] = row_ok ? __builtin_bit_cast(i16x8_t, *(const uint4*)(qp + 16 * kk + 8 * g))
                      : i16x8_t{0, 0, 0, 0, 0, 0, 0, 0};
  }

  const int ks = s * L;
  const int ke = min(Nk, ks + L);
  const int nst = (ke - ks + kSkStage - 1) / kSkStage;
  const size_t kv_off = (size_t)bkv * Nk * D;
  const uint32_t head_bytes = (uint32_t)Nk * D * 2;
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(K + kv_off, head_bytes);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(V + kv_off, head_bytes);
  // lane's byte offset within a stage for piece i: LDS chunk (r, c) holds logical chunk c ^ swz(r)
  uint32_t goff[PIECES];
#pragma unroll
  for (int i = 0; i < PIECES; ++i) {
    const int p = 64 * i + lane;
    const int r = p / CH, pch = p % CH;
    goff[i] = ((uint32_t)r * D + ((pch ^ swz<D>(r)) << 3)) * 2;
  }
  auto load_stage = [&](int j, auto sl) __attribute__((always_inline)) {
    const uint32_t base = (uint32_t)(ks + j * kSkStage) * D * 2;
    short* kd = slot(sl);
#pragma unroll
    for (int i = 0; i < PIECES; ++i) {
      buffer_load16_lds(krs, kd + 512 * i, goff[i], base);
      buffer_load16_lds(vrs, kd + STAGE + 512 * i, goff[i], base);
    }
  };
  int off_k[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) off_k[kk] = chunk_index<D>(l32, 2 * kk + g) * 8;
  int off_v[DB][2];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) off_v[db][hh] = tr_off<D>(lane, db, hh);

  f32x16_t o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x16_t{};
  float m = -INFINITY, l = 0.f;

  // keys below klim are visible to every row (none past Nk, none after a row's causal position)
  const int klim = min(ke, CAUSAL ? Nk - Nq + 1 : Nk);
  auto stage = [&](int j, auto sl) __attribute__((always_inline)) {
    constexpr int SL = decltype(sl)::value;
    // stages j .. j + ahead are in flight, j the oldest: wait for it (and for the LDS reads of
    // stage j - 1, whose slot the next request overwrites)
    const int ahead = min(kSkSlots - 2, nst - 1 - j);
    if (ahead >= 2) wait_vmem_lds<2 * LPS>();
    else if (ahead == 1) wait_vmem_lds<LPS>();
    else wait_vmem_lds<0>();
    if (j + kSkSlots - 1 < nst) load_stage(j + kSkSlots - 1, std::integral_constant<int, (SL + kSkSlots - 1) % kSkSlots>{});
    const short* Kb = slot(sl);
    const short* Vb = Kb + STAGE;
    f32x16_t st = f32x16_t{};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const i16x8_t a = __builtin_bit_cast(i16x8_t, *(const uint4*)(Kb + off_k[kk]));
      st = mfma32x32x16<BF16>(a, qf[kk], st);
    }
    const int kw0 = ks + j * kSkStage;
    if (kw0 + kSkStage > klim) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kw0 + 8 * (r >> 2) + 4 * g + (r & 3);
        if (key >= ke || (CAUSAL && key > qpos)) st[r] = -INFINITY;
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, st[r]);
    const float mt = fmaxf(m, max_halves(mx) * c);
    const float alpha = (m == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m - mt);
    const float muse = (mt == -INFINITY) ? 0.f : mt;
    float rs = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = __builtin_amdgcn_exp2f(st[r] * c - muse);
      st[r] = p;
      rs += p;
    }
    m = mt;
    l = l * alpha + rs;
    // the accumulator changes only where a row's maximum grew (alpha = 1 leaves it as it is)
    if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] *= alpha;
    }
    const i16x8_t pf[2] = {pack8<BF16>(st, 0), pack8<BF16>(st, 8)};
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] = mfma32x32x16<BF16>(read_tr8(Vb + 16 * t * D, off_v[db]), pf[t], o[db]);
  };

  if (nst > 0) load_stage(0, S0{});
  if (nst > 1) load_stage(1, S1{});
  if (nst > 2) load_stage(2, S2{});
  for (int j = 0; j < nst; j += kSkSlots) {
    stage(j, S0{});
    if (j + 1 >= nst) break;
    stage(j + 1, S1{});
    if (j + 2 >= nst) break;
    stage(j + 2, S2{});
    if (j + 3 >= nst) break;
    stage(j + 3, S3{});
  }

  // the two halves of the wave hold different keys of the same rows and the same maximum
  const float lt = sum_halves(l);
  if (row_ok) {
    const size_t prow = (size_t)s * B * Hq * Nq + ((size_t)b * Hq + hq) * Nq + qi;
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    float* op = Opart + prow * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const float4 val = {o[db][4 * q4] * inv, o[db][4 * q4 + 1] * inv, o[db][4 * q4 + 2] * inv,
                            o[db][4 * q4 + 3] * inv};
        *(float4*)(op + 32 * db + 8 * q4 + 4 * g) = val;
      }
    if (g == 0) Lpart[prow] = lt > 0.f ? (m + __log2f(lt)) * kLn2 : -INFINITY;
  }
}

// Sum and maximum over the 64 lanes of a wave (a fixed butterfly order: every lane gets the same
// value, and the result does not depend on the launch).
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m);
  return x;
}

// One wave per output row: LSE = ln sum_s exp(LSE_s), O = sum_s exp(LSE_s - LSE) O_s.  The lanes
// read the splits' logsumexps 64 at a time (lane i holds split c + i of a chunk and its weight);
// lane l then accumulates elements 2l and 2l + 1 over the splits in order, each split's weight
// broadcast from the lane that holds it, the loads of 16 splits in flight together (lanes >=
// D / 2 only take part in the logsumexp).
template <bool BF16, int D>
__global__ __launch_bounds__(256) void fwd_split_merge_kernel(const float* __restrict__ Opart,
                                                              const float* __restrict__ Lpart, uint16_t* __restrict__ O,
                                                              float* __restrict__ LSE, int rows, int S) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  // the first 64 logsumexps are loaded once, for the maximum and for the weights; the first 16
  // splits' partial outputs are requested at the same time (they do not depend on the weights)
  const float ls0 = lane < S ? Lpart[(size_t)lane * rows + row] : -INFINITY;
  const bool act = lane < D / 2;
  const size_t step = (size_t)rows * D;             // floats from one split's row to the next's
  const int n0 = min(64, S);
  float2 ov0[16];
#pragma unroll
  for (int u = 0; u < 16; ++u)
    ov0[u] = act ? *(const float2*)(Opart + (size_t)row * D + 2 * lane + (size_t)min(u, n0 - 1) * step)
                 : float2{0.f, 0.f};
  float mx = ls0;
  for (int s = lane + 64; s < S; s += 64) mx = fmaxf(mx, Lpart[(size_t)s * rows + row]);
  mx = wave_max(mx);
  float a0 = 0.f, a1 = 0.f, wpart = 0.f;
  auto weight = [](float w, int i) __attribute__((always_inline)) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), i));
  };
  for (int c = 0; c < S; c += 64) {
    const float ls = c == 0 ? ls0 : (c + lane < S ? Lpart[(size_t)(c + lane) * rows + row] : -INFINITY);
    const float wgt = (ls == -INFINITY) ? 0.f : __expf(ls - mx);
    wpart += wgt;
    const int n = min(64, S - c);
    const float* op = Opart + ((size_t)c * rows + row) * D + 2 * lane;
    // batches of 16 splits with their loads in flight together; past the chunk's last split the
    // index stays on that split and the weight (held by a lane past S) is zero
    for (int i = 0; i < n; i += 16) {
      float2 ov[16];
      if (c == 0 && i == 0) {
#pragma unroll
        for (int u = 0; u < 16; ++u) ov[u] = ov0[u];
      } else {
#pragma unroll
        for (int u = 0; u < 16; ++u)
          ov[u] = act ? *(const float2*)(op + (size_t)min(i + u, n - 1) * step) : float2{0.f, 0.f};
      }
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const float w = weight(wgt, i + u);
        a0 += w * ov[u].x;
        a1 += w * ov[u].y;
      }
    }
  }
  const float wsum = wave_sum(wpart);
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  if (act) *(uint32_t*)(O + (size_t)row * D + 2 * lane) = pack2<BF16>(a0 * inv, a1 * inv);
  if (lane == 0) LSE[row] = wsum > 0.f ? mx + __logf(wsum) : -INFINITY;
}

template <bool BF16, int D, bool CAUSAL>
static hipError_t launch_split_t(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
                                 int Hkv, int Nq, int Nk, float scale, int num_splits, void* workspace,
                                 hipStream_t stream) {
  int S, L;
  splitkv_plan(B, Hq, Hkv, Nq, Nk, num_splits, &S, &L);
  const size_t rows = (size_t)B * Hq * Nq;
  const int RG = splitkv_row_groups(Hq, Hkv, Nq);
  float* opart = (float*)workspace;
  float* lpart = (float*)((char*)workspace + ((size_t)S * rows * D * 4 + 255) / 256 * 256);
  hipLaunchKernelGGL((fwd_split_kernel<BF16, D, CAUSAL>), dim3((unsigned)(B * Hkv * S * RG)), dim3(64), 0, stream,
                     (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, opart, lpart, B, Hq, Hkv, Nq, Nk,
                     S, L, scale * kLog2e);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((fwd_split_merge_kernel<BF16, D>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream,
                     (const float*)opart, (const float*)lpart, (uint16_t*)o, lse, (int)rows, S);
  return hipGetLastError();
}

hipError_t launch_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
                              int Hkv, int Nq, int Nk, int d, bool causal, float scale, bool bf16, int num_splits,
                              void* workspace, hipStream_t stream) {
#define EAO_SPLIT(BF, DD, CA) \
  return launch_split_t<BF, DD, CA>(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, scale, num_splits, workspace, stream)
  if (bf16) {
    if (d == 128) { if (causal) EAO_SPLIT(true, 128, true); else EAO_SPLIT(true, 128, false); }
    else { if (causal) EAO_SPLIT(true, 64, true); else EAO_SPLIT(true, 64, false); }
  } else {
    if (d == 128) { if (causal) EAO_SPLIT(false, 128, true); else EAO_SPLIT(false, 128, false); }
    else { if (causal) EAO_SPLIT(false, 64, true); else EAO_SPLIT(false, 64, false); }
  }
#undef EAO_SPLIT
}

}  // namespace eao
