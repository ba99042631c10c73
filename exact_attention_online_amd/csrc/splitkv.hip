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
//   * split kernel: one workgroup of 4 waves per (batch, K/V head, split, group of 32 rows).
//     The query rows that use the K/V head -- G = Hq / Hkv heads times Nq rows -- are taken 32 at
//     a time as the 32 columns of one MFMA tile (transposed formulation as in the main forward:
//     a lane owns one row); the workgroups of one split's row groups are adjacent in the grid,
//     so beyond the first they find the split's keys in L2.  Key
//     tiles of 128 go straight from HBM into double-buffered LDS (direct buffer -> LDS loads);
//     each wave takes its own 32 keys of every tile and keeps its own running max, sum and
//     O^T, so the four waves stream disjoint keys and are merged once, through LDS, at the end.
//     The kernel is bound by HBM bandwidth (every key is read once per K/V head).
//   * merge kernel: one wave per output row.
//
// Causal alignment for Nq < Nk (bottom-right): query i sits at position Nk - Nq + i and sees
// keys j <= Nk - Nq + i.
#include <atomic>
#include <mutex>

#include "common.hpp"

namespace eao {

constexpr int kSkTile = 128;   // keys per tile (32 per wave)

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
    // about two workgroups per compute unit, but splits of at least 8 tiles: shorter splits
    // spend more time in their prologue and the merge than they save
    const int wg = B * Hkv * splitkv_row_groups(Hq, Hkv, Nq);
    const int want = (2 * 256 + wg - 1) / wg;
    s = want < tiles / 8 ? want : tiles / 8;
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
__global__ __launch_bounds__(256, 1) void fwd_split_kernel(const uint16_t* __restrict__ Q,
                                                           const uint16_t* __restrict__ K,
                                                           const uint16_t* __restrict__ V, float* __restrict__ Opart,
                                                           float* __restrict__ Lpart, int B, int Hq, int Hkv, int Nq,
                                                           int Nk, int S, int L, float c /* scale * log2(e) */) {
  constexpr int CH = D / 8, KK = D / 16, DB = D / 32;
  constexpr int TILE = kSkTile * D;                 // 16-bit elements per K or V tile
  constexpr int PIECES = TILE * 2 / 1024;           // 1 KB direct-load pieces per tile
  static_assert(PIECES % 4 == 0, "each wave moves the same number of pieces");
  __shared__ __attribute__((aligned(1024))) short k_lds0[TILE];
  __shared__ __attribute__((aligned(1024))) short k_lds1[TILE];
  __shared__ __attribute__((aligned(1024))) short v_lds0[TILE];
  __shared__ __attribute__((aligned(1024))) short v_lds1[TILE];
  __shared__ float red_m[4][32], red_l[4][32];
  auto Ks = [&](auto par) -> short* __attribute__((always_inline)) {
    if constexpr (decltype(par)::value == 0) return k_lds0; else return k_lds1;
  };
  auto Vs = [&](auto par) -> short* __attribute__((always_inline)) {
    if constexpr (decltype(par)::value == 0) return v_lds0; else return v_lds1;
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, g = lane >> 5, l32 = lane & 31;
  const int G16 = lane >> 4, li = lane & 15;
  const int G = Hq / Hkv, R = G * Nq, RG = (R + 31) / 32;
  const int rg = blockIdx.x % RG, s = (blockIdx.x / RG) % S, bkv = blockIdx.x / (RG * S);
  const int b = bkv / Hkv, kvh = bkv % Hkv;
  const int r0 = 32 * rg;                           // first row of this workgroup's group
  // this lane's query row: head kvh * G + row / Nq, row row % Nq (rows >= R are padding)
  const int row = r0 + l32;
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
  const int ntiles = (ke - ks + kSkTile - 1) / kSkTile;
  const size_t kv_off = (size_t)bkv * Nk * D;
  const uint32_t head_bytes = (uint32_t)Nk * D * 2;
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(K + kv_off, head_bytes);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(V + kv_off, head_bytes);
  uint32_t goff[PIECES / 4];
#pragma unroll
  for (int i = 0; i < PIECES / 4; ++i) {
    const int p = 64 * (4 * i + w) + lane;
    const int r = p / CH, pch = p % CH;
    goff[i] = ((uint32_t)r * D + ((pch ^ swz<D>(r)) << 3)) * 2;
  }
  auto load_tile = [&](int j, auto par) __attribute__((always_inline)) {
    const uint32_t base = (uint32_t)(ks + j * kSkTile) * D * 2;
    short* kd = Ks(par);
    short* vd = Vs(par);
#pragma unroll
    for (int i = 0; i < PIECES / 4; ++i) {
      buffer_load16_lds(krs, kd + 512 * (4 * i + w), goff[i] + base);
      buffer_load16_lds(vrs, vd + 512 * (4 * i + w), goff[i] + base);
    }
  };
  int off_k[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) off_k[kk] = (32 * w) * D + chunk_index<D>(l32, 2 * kk + g) * 8;
  int off_v[DB][2];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
      off_v[db][hh] = (32 * w) * D +
                      elem_index<D>(4 * (G16 >> 1) + (li >> 2) + 8 * hh, 32 * db + 16 * (G16 & 1) + 4 * (li & 3));

  f32x16_t o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x16_t{};
  float m = -INFINITY, l = 0.f;

  // tiles that may hold keys a row cannot see (past Nk, or after its causal position)
  const int limit = CAUSAL ? Nk - Nq + 1 : Nk;      // keys below this are visible to every row
  auto tile = [&](int j, auto par, auto mask_tag) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    using Other = std::integral_constant<int, 1 - decltype(par)::value>;
    if (j + 1 < ntiles) load_tile(j + 1, Other{});
    const short* Kb = Ks(par);
    const short* Vb = Vs(par);
    f32x16_t st = f32x16_t{};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const i16x8_t a = __builtin_bit_cast(i16x8_t, *(const uint4*)(Kb + off_k[kk]));
      st = mfma32x32x16<BF16>(a, qf[kk], st);
    }
    const int kw0 = ks + j * kSkTile + 32 * w;      // this wave's first key
    if constexpr (MASK) {
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
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] *= alpha;
    const i16x8_t pf[2] = {pack8<BF16>(st, 0), pack8<BF16>(st, 8)};
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const i16x4_t lo = ds_read_tr16(Vb + 16 * t * D + off_v[db][0]);
        const i16x4_t hi = ds_read_tr16(Vb + 16 * t * D + off_v[db][1]);
        const i16x8_t a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        o[db] = mfma32x32x16<BF16>(a, pf[t], o[db]);
      }
    wait_all_loads();
    __syncthreads();
  };

  if (ntiles > 0) load_tile(0, Par0{});
  wait_all_loads();
  __syncthreads();
  // tiles [0, jmask) lie wholly below `limit`
  const int jmask = min(ntiles, max(0, (limit - ks) / kSkTile));
  int j = 0;
  for (; j + 1 < jmask; j += 2) {
    tile(j, Par0{}, std::false_type{});
    tile(j + 1, Par1{}, std::false_type{});
  }
  if (j < jmask) {
    tile(j, Par0{}, std::false_type{});
    ++j;
  }
  for (; j < ntiles; ++j) {
    if (j & 1) tile(j, Par1{}, std::true_type{});
    else tile(j, Par0{}, std::true_type{});
  }

  // merge the four waves (disjoint keys, same rows): M = max m_w, L = sum l_w 2^(m_w - M),
  // O = sum O_w 2^(m_w - M) / L; the K/V buffers are free now and hold the four O^T
  const float lt = sum_halves(l);
  if (g == 0) {
    red_m[w][l32] = m;
    red_l[w][l32] = lt;
  }
  __syncthreads();
  float mall = -INFINITY;
#pragma unroll
  for (int ww = 0; ww < 4; ++ww) mall = fmaxf(mall, red_m[ww][l32]);
  const float fw = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m - mall);
  // [2 waves][32 rows][D] fp32 fills one K (waves 0, 1) or V (waves 2, 3) buffer exactly
  static_assert(2 * 32 * D * 4 == TILE * 2, "two waves' O^T fill one tile buffer");
  float* ost_k = (float*)k_lds0;
  float* ost_v = (float*)v_lds0;
  float* ost = (w < 2 ? ost_k : ost_v) + (w & 1) * 32 * D;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int d = 32 * db + 8 * (r >> 2) + 4 * g + (r & 3);
      ost[l32 * D + d] = o[db][r] * fw;
    }
  __syncthreads();
  // 256 threads x (32 rows x D) / 256 outputs each; rows >= R are not written
  const size_t prow0 = (size_t)s * B * Hq * Nq;      // partial rows of split s
  for (int e = tid; e < 32 * D; e += 256) {
    const int rr = e / D, d = e % D;
    if (r0 + rr >= R) continue;
    float mtot = -INFINITY, ltot = 0.f;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) mtot = fmaxf(mtot, red_m[ww][rr]);
    float sum = 0.f;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      const float mw = red_m[ww][rr];
      const float f = (mw == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mw - mtot);
      ltot += red_l[ww][rr] * f;
      sum += (ww < 2 ? ost_k : ost_v)[((ww & 1) * 32 + rr) * D + d];
    }
    const int ghh = (r0 + rr) / Nq, qq = (r0 + rr) % Nq;
    const size_t prow = prow0 + ((size_t)b * Hq + kvh * G + ghh) * Nq + qq;
    Opart[prow * D + d] = ltot > 0.f ? sum / ltot : 0.f;
    if (d == 0) Lpart[prow] = ltot > 0.f ? (mtot + __log2f(ltot)) * kLn2 : -INFINITY;
  }
}

// One wave per output row: LSE = ln sum_s exp(LSE_s), O = sum_s exp(LSE_s - LSE) O_s; lane l
// handles elements 2l and 2l + 1 (lanes >= D / 2 only join the LSE).
template <bool BF16, int D>
__global__ __launch_bounds__(256) void fwd_split_merge_kernel(const float* __restrict__ Opart,
                                                              const float* __restrict__ Lpart, uint16_t* __restrict__ O,
                                                              float* __restrict__ LSE, int rows, int S) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  float mx = -INFINITY;
  for (int s = 0; s < S; ++s) mx = fmaxf(mx, Lpart[(size_t)s * rows + row]);
  const bool act = lane < D / 2;
  float a0 = 0.f, a1 = 0.f, wsum = 0.f;
  for (int s = 0; s < S; ++s) {
    const float ls = Lpart[(size_t)s * rows + row];
    const float wgt = (ls == -INFINITY) ? 0.f : __expf(ls - mx);
    wsum += wgt;
    if (act) {
      const float2 ov = *(const float2*)(Opart + ((size_t)s * rows + row) * D + 2 * lane);
      a0 += wgt * ov.x;
      a1 += wgt * ov.y;
    }
  }
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
  hipLaunchKernelGGL((fwd_split_kernel<BF16, D, CAUSAL>), dim3((unsigned)(B * Hkv * S * RG)), dim3(256), 0, stream,
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
