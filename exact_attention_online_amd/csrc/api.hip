// extern "C" entry points of libattn.so: argument checks on the host, then kernel dispatch.
// Every check runs before any HIP call, so a rejected call enqueues nothing (and works on a
// machine without a GPU).
#include <math.h>
#include <stdint.h>

#include <initializer_list>

#include "../../include/attn.h"
#include "common.hpp"

namespace eao {
hipError_t launch_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv,
                      int N, int d, bool causal, float scale, bool bf16, hipStream_t stream);
hipError_t launch_bwd_pre(const void* q, const void* k, const void* o, const void* dout, const float* lse, int B,
                          int Hq, int Hkv, int N, int d, bool bf16, void* workspace, hipStream_t stream,
                          int max_seqlen = 0, const int* cu = nullptr);
hipError_t launch_bwd_dkdv(const void* q, const void* k, const void* v, const void* dout, const float* lse, void* dk,
                           void* dv, int B, int Hq, int Hkv, int N, int d, bool causal, float scale, bool bf16,
                           bool out32, const void* workspace, hipStream_t stream, int max_seqlen = 0,
                           const int* cu = nullptr);
hipError_t launch_bwd_dq(const void* q, const void* k, const void* v, const void* dout, const float* lse, void* dq,
                         int B, int Hq, int Hkv, int N, int d, bool causal, float scale, bool bf16, bool out32,
                         const void* workspace, hipStream_t stream, int max_seqlen = 0, const int* cu = nullptr);
hipError_t launch_bwd_dkdv_ext(const void* q, const void* k, const void* v, const void* dout, const float* lse,
                               void* dk, void* dv, int B, int Hq, int Hkv, int N, int d, bool causal, float scale,
                               bool bf16, bool out32, const void* workspace, hipStream_t stream, int window,
                               const float* slopes);
hipError_t launch_bwd_dq_ext(const void* q, const void* k, const void* v, const void* dout, const float* lse,
                             void* dq, int B, int Hq, int Hkv, int N, int d, bool causal, float scale, bool bf16,
                             bool out32, const void* workspace, hipStream_t stream, int window, const float* slopes);
hipError_t launch_fwd_ext(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv,
                          int N, int d, bool causal, float scale, bool bf16, int window, const float* slopes,
                          hipStream_t stream);
hipError_t launch_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse, const int* cu_seqlens,
                             int B, int Hq, int Hkv, int T, int max_seqlen, int d, bool causal, float scale,
                             bool bf16, hipStream_t stream);
hipError_t launch_fp8_prep(const float* x, uint8_t* x8, float* descale, const int8_t* signs, int B, int H, int N,
                           int d, bool pow2, hipStream_t stream);
hipError_t launch_fwd_fp8(const uint8_t* q, const uint8_t* k, const uint8_t* v, uint16_t* o, float* lse,
                          const float* qs, const float* ks, const float* vs, int B, int Hq, int Hkv, int N, int d,
                          bool causal, float scale, hipStream_t stream);
size_t bwd_workspace_bytes(int B, int Hq, int Hkv, int N, int d, bool dense);
hipError_t launch_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
                              int Hkv, int Nq, int Nk, int d, bool causal, float scale, bool bf16, int num_splits,
                              void* workspace, hipStream_t stream);
size_t splitkv_workspace_bytes(int B, int Hq, int Hkv, int Nq, int Nk, int d, int num_splits);
hipError_t launch_clock_probe(unsigned long long* out, int groups, long long ticks, hipStream_t stream);
hipError_t launch_mfma_probe(const void* data, size_t n, bool fp8, float* out, int groups, int iters,
                             hipStream_t stream);
hipError_t launch_hbm_probe(const uint8_t* data, uint32_t share, uint32_t* out, int groups, hipStream_t stream);
size_t splitkv_scratch_bytes();
hipError_t splitkv_scratch_address(void** out);
}  // namespace eao

namespace {

bool aligned16(const void* p) { return p != nullptr && ((uintptr_t)p & 15u) == 0; }

// Common shape checks; returns ATTN_OK or the status to report.
int check_sizes(int B, int Hq, int Hkv, int N, int d) {
  if (B < 1 || Hq < 1 || Hkv < 1 || N < 1 || d < 1) return ATTN_ERR_INVALID;
  if (Hq % Hkv != 0) return ATTN_ERR_INVALID;
  // element counts must fit the kernels' 64-bit offsets and the 32-bit grid
  const double elems = (double)B * Hq * N * d;
  if (elems > 9.0e15) return ATTN_ERR_INVALID;
  if ((double)B * Hq * ((N + 127) / 128) > 2.0e9) return ATTN_ERR_UNSUPPORTED;
  if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
  // one head of one tensor is addressed with 32-bit byte offsets
  if ((double)N * d * 4 > 2147483647.0) return ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

bool scale_ok(float s) { return isfinite(s) && s > 0.f; }

}  // namespace

extern "C" {

const char* attn_status_string(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_INVALID: return "invalid argument (null or misaligned pointer, bad size, scale or dtype)";
    case ATTN_ERR_UNSUPPORTED: return "unsupported configuration (head dim must be 64 or 128)";
    case ATTN_ERR_WORKSPACE: return "workspace missing or too small";
    case ATTN_ERR_HIP: return "HIP runtime error at launch";
    case ATTN_ERR_SCRATCH: return "problem needs more than the static scratch of the allocation-free entry point (8 MiB)";
    default: return "unknown status";
  }
}

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv, int N, int d,
             int causal, float softmax_scale, int dtype, const float* q_descale, const float* k_descale,
             const float* v_descale, attn_stream_t stream) {
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse)) return ATTN_ERR_INVALID;
  if (!scale_ok(softmax_scale)) return ATTN_ERR_INVALID;
  if (dtype != ATTN_F16 && dtype != ATTN_BF16 && dtype != ATTN_FP8_E4M3) return ATTN_ERR_INVALID;
  const int st = check_sizes(B, Hq, Hkv, N, d);
  if (st != ATTN_OK) return st;
  hipError_t e;
  if (dtype == ATTN_FP8_E4M3) {
    if (!aligned16(q_descale) || !aligned16(k_descale) || !aligned16(v_descale)) return ATTN_ERR_INVALID;
    if (d != 128) return ATTN_ERR_UNSUPPORTED;
    e = eao::launch_fwd_fp8((const uint8_t*)q, (const uint8_t*)k, (const uint8_t*)v, (uint16_t*)o, lse, q_descale,
                            k_descale, v_descale, B, Hq, Hkv, N, d, causal != 0, softmax_scale,
                            (hipStream_t)stream);
  } else {
    if (q_descale || k_descale || v_descale) return ATTN_ERR_INVALID;
    e = eao::launch_fwd(q, k, v, o, lse, B, Hq, Hkv, N, d, causal != 0, softmax_scale, dtype == ATTN_BF16,
                        (hipStream_t)stream);
  }
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

int attn_fwd_ext(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv, int N,
                 int d, int causal, float softmax_scale, int dtype, int window, const float* alibi_slopes,
                 attn_stream_t stream) {
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse)) return ATTN_ERR_INVALID;
  if (!scale_ok(softmax_scale) || window < 0) return ATTN_ERR_INVALID;
  if (alibi_slopes != nullptr && ((uintptr_t)alibi_slopes & 3u) != 0) return ATTN_ERR_INVALID;
  if (dtype != ATTN_F16 && dtype != ATTN_BF16) return dtype == ATTN_FP8_E4M3 ? ATTN_ERR_UNSUPPORTED : ATTN_ERR_INVALID;
  const int st = check_sizes(B, Hq, Hkv, N, d);
  if (st != ATTN_OK) return st;
  return eao::launch_fwd_ext(q, k, v, o, lse, B, Hq, Hkv, N, d, causal != 0, softmax_scale, dtype == ATTN_BF16,
                             window, alibi_slopes, (hipStream_t)stream) == hipSuccess
             ? ATTN_OK : ATTN_ERR_HIP;
}

int attn_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse, const int* cu_seqlens, int B,
                    int Hq, int Hkv, int T, int max_seqlen, int d, int causal, float softmax_scale, int dtype,
                    attn_stream_t stream) {
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse)) return ATTN_ERR_INVALID;
  if (cu_seqlens == nullptr || ((uintptr_t)cu_seqlens & 3u) != 0) return ATTN_ERR_INVALID;
  if (!scale_ok(softmax_scale) || max_seqlen < 1 || max_seqlen > T) return ATTN_ERR_INVALID;
  if (dtype != ATTN_F16 && dtype != ATTN_BF16) return dtype == ATTN_FP8_E4M3 ? ATTN_ERR_UNSUPPORTED : ATTN_ERR_INVALID;
  // the packed tensors are one batch of T rows per head
  int st = check_sizes(1, Hq, Hkv, T, d);
  if (st != ATTN_OK) return st;
  if (B < 1 || (double)B * Hq * ((max_seqlen + 127) / 128) > 2.0e9) return ATTN_ERR_INVALID;
  return eao::launch_fwd_varlen(q, k, v, o, lse, cu_seqlens, B, Hq, Hkv, T, max_seqlen, d, causal != 0,
                                softmax_scale, dtype == ATTN_BF16, (hipStream_t)stream) == hipSuccess
             ? ATTN_OK : ATTN_ERR_HIP;
}

size_t attn_bwd_workspace_size(int B, int Hq, int Hkv, int N, int d) {
  if (check_sizes(B, Hq, Hkv, N, d) != ATTN_OK) return 0;
  return eao::bwd_workspace_bytes(B, Hq, Hkv, N, d, true);
}

// Shared checks of the backward entry points (pointer list, sizes, scale, dtype, workspace).
static int check_bwd(std::initializer_list<const void*> ptrs, int B, int Hq, int Hkv, int N, int d, float scale,
                     int dtype, int grad_dtype, const void* workspace, size_t workspace_bytes) {
  for (const void* p : ptrs)
    if (!aligned16(p)) return ATTN_ERR_INVALID;
  if (!scale_ok(scale)) return ATTN_ERR_INVALID;
  if (dtype != ATTN_F16 && dtype != ATTN_BF16) return dtype == ATTN_FP8_E4M3 ? ATTN_ERR_UNSUPPORTED : ATTN_ERR_INVALID;
  if (grad_dtype != dtype && grad_dtype != ATTN_F32) return ATTN_ERR_INVALID;
  const int st = check_sizes(B, Hq, Hkv, N, d);
  if (st != ATTN_OK) return st;
  if (workspace == nullptr || ((uintptr_t)workspace & 255u) != 0) return ATTN_ERR_WORKSPACE;
  if (workspace_bytes < eao::bwd_workspace_bytes(B, Hq, Hkv, N, d, true)) return ATTN_ERR_WORKSPACE;
  return ATTN_OK;
}

int attn_bwd_preprocess(const void* q, const void* k, const void* o, const void* dout, const float* lse, int B,
                        int Hq, int Hkv, int N, int d, int dtype, void* workspace, size_t workspace_bytes,
                        attn_stream_t stream) {
  const int st = check_bwd({q, k, o, dout, lse}, B, Hq, Hkv, N, d, 1.f, dtype, dtype, workspace, workspace_bytes);
  if (st != ATTN_OK) return st;
  return eao::launch_bwd_pre(q, k, o, dout, lse, B, Hq, Hkv, N, d, dtype == ATTN_BF16, workspace,
                             (hipStream_t)stream) == hipSuccess
             ? ATTN_OK : ATTN_ERR_HIP;
}

int attn_bwd_dkdv(const void* q, const void* k, const void* v, const void* dout, const float* lse, void* dk, void* dv,
                  int B, int Hq, int Hkv, int N, int d, int causal, float softmax_scale, int dtype, int grad_dtype,
                  const void* workspace, size_t workspace_bytes, attn_stream_t stream) {
  const int st = check_bwd({q, k, v, dout, lse, dk, dv}, B, Hq, Hkv, N, d, softmax_scale, dtype, grad_dtype,
                           workspace, workspace_bytes);
  if (st != ATTN_OK) return st;
  return eao::launch_bwd_dkdv(q, k, v, dout, lse, dk, dv, B, Hq, Hkv, N, d, causal != 0, softmax_scale,
                              dtype == ATTN_BF16, grad_dtype == ATTN_F32, workspace, (hipStream_t)stream) == hipSuccess
             ? ATTN_OK : ATTN_ERR_HIP;
}

int attn_bwd_dq(const void* q, const void* k, const void* v, const void* dout, const float* lse, void* dq, int B,
                int Hq, int Hkv, int N, int d, int causal, float softmax_scale, int dtype, int grad_dtype,
                const void* workspace, size_t workspace_bytes, attn_stream_t stream) {
  const int st = check_bwd({q, k, v, dout, lse, dq}, B, Hq, Hkv, N, d, softmax_scale, dtype, grad_dtype, workspace,
                           workspace_bytes);
  if (st != ATTN_OK) return st;
  return eao::launch_bwd_dq(q, k, v, dout, lse, dq, B, Hq, Hkv, N, d, causal != 0, softmax_scale,
                            dtype == ATTN_BF16, grad_dtype == ATTN_F32, workspace, (hipStream_t)stream) == hipSuccess
             ? ATTN_OK : ATTN_ERR_HIP;
}

int attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse, void* dq,
             void* dk, void* dv, int B, int Hq, int Hkv, int N, int d, int causal, float softmax_scale, int dtype,
             int grad_dtype, void* workspace, size_t workspace_bytes, attn_stream_t stream) {
  const int st = check_bwd({q, k, v, o, dout, lse, dq, dk, dv}, B, Hq, Hkv, N, d, softmax_scale, dtype, grad_dtype,
                           workspace, workspace_bytes);
  if (st != ATTN_OK) return st;
  const bool bf16 = dtype == ATTN_BF16, out32 = grad_dtype == ATTN_F32;
  const hipStream_t s = (hipStream_t)stream;
  if (eao::launch_bwd_pre(q, k, o, dout, lse, B, Hq, Hkv, N, d, bf16, workspace, s) != hipSuccess) return ATTN_ERR_HIP;
  if (eao::launch_bwd_dkdv(q, k, v, dout, lse, dk, dv, B, Hq, Hkv, N, d, causal != 0, softmax_scale, bf16, out32,
                           workspace, s) != hipSuccess)
    return ATTN_ERR_HIP;
  if (eao::launch_bwd_dq(q, k, v, dout, lse, dq, B, Hq, Hkv, N, d, causal != 0, softmax_scale, bf16, out32,
                         workspace, s) != hipSuccess)
    return ATTN_ERR_HIP;
  return ATTN_OK;
}

int attn_bwd_ext(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                 void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int N, int d, int causal, float softmax_scale,
                 int dtype, int grad_dtype, int window, const float* alibi_slopes, void* workspace,
                 size_t workspace_bytes, attn_stream_t stream) {
  const int st = check_bwd({q, k, v, o, dout, lse, dq, dk, dv}, B, Hq, Hkv, N, d, softmax_scale, dtype, grad_dtype,
                           workspace, workspace_bytes);
  if (st != ATTN_OK) return st;
  if (window < 0) return ATTN_ERR_INVALID;
  if (alibi_slopes != nullptr && ((uintptr_t)alibi_slopes & 3u) != 0) return ATTN_ERR_INVALID;
  const bool bf16 = dtype == ATTN_BF16, out32 = grad_dtype == ATTN_F32;
  const hipStream_t s = (hipStream_t)stream;
  if (eao::launch_bwd_pre(q, k, o, dout, lse, B, Hq, Hkv, N, d, bf16, workspace, s) != hipSuccess) return ATTN_ERR_HIP;
  if (eao::launch_bwd_dkdv_ext(q, k, v, dout, lse, dk, dv, B, Hq, Hkv, N, d, causal != 0, softmax_scale, bf16, out32,
                               workspace, s, window, alibi_slopes) != hipSuccess)
    return ATTN_ERR_HIP;
  if (eao::launch_bwd_dq_ext(q, k, v, dout, lse, dq, B, Hq, Hkv, N, d, causal != 0, softmax_scale, bf16, out32,
                             workspace, s, window, alibi_slopes) != hipSuccess)
    return ATTN_ERR_HIP;
  return ATTN_OK;
}

size_t attn_bwd_varlen_workspace_size(int B, int Hq, int Hkv, int max_seqlen, int d) {
  if (check_sizes(B, Hq, Hkv, max_seqlen, d) != ATTN_OK) return 0;
  return eao::bwd_workspace_bytes(B, Hq, Hkv, max_seqlen, d, false);
}

int attn_bwd_varlen(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                    void* dq, void* dk, void* dv, const int* cu_seqlens, int B, int Hq, int Hkv, int T,
                    int max_seqlen, int d, int causal, float softmax_scale, int dtype, int grad_dtype,
                    void* workspace, size_t workspace_bytes, attn_stream_t stream) {
  for (const void* p : {q, k, v, o, dout, (const void*)lse, (const void*)dq, (const void*)dk, (const void*)dv})
    if (!aligned16(p)) return ATTN_ERR_INVALID;
  if (cu_seqlens == nullptr || ((uintptr_t)cu_seqlens & 3u) != 0) return ATTN_ERR_INVALID;
  if (!scale_ok(softmax_scale) || max_seqlen < 1 || max_seqlen > T) return ATTN_ERR_INVALID;
  if (dtype != ATTN_F16 && dtype != ATTN_BF16) return dtype == ATTN_FP8_E4M3 ? ATTN_ERR_UNSUPPORTED : ATTN_ERR_INVALID;
  if (grad_dtype != dtype && grad_dtype != ATTN_F32) return ATTN_ERR_INVALID;
  // the packed tensors are one batch of T rows per head; the workspace is B sequences of max_seqlen
  int st = check_sizes(1, Hq, Hkv, T, d);
  if (st != ATTN_OK) return st;
  st = check_sizes(B, Hq, Hkv, max_seqlen, d);
  if (st != ATTN_OK) return st;
  if (workspace == nullptr || ((uintptr_t)workspace & 255u) != 0) return ATTN_ERR_WORKSPACE;
  if (workspace_bytes < eao::bwd_workspace_bytes(B, Hq, Hkv, max_seqlen, d, false)) return ATTN_ERR_WORKSPACE;
  const bool bf16 = dtype == ATTN_BF16, out32 = grad_dtype == ATTN_F32;
  const hipStream_t s = (hipStream_t)stream;
  if (eao::launch_bwd_pre(q, k, o, dout, lse, B, Hq, Hkv, T, d, bf16, workspace, s, max_seqlen, cu_seqlens) !=
      hipSuccess)
    return ATTN_ERR_HIP;
  if (eao::launch_bwd_dkdv(q, k, v, dout, lse, dk, dv, B, Hq, Hkv, T, d, causal != 0, softmax_scale, bf16, out32,
                           workspace, s, max_seqlen, cu_seqlens) != hipSuccess)
    return ATTN_ERR_HIP;
  if (eao::launch_bwd_dq(q, k, v, dout, lse, dq, B, Hq, Hkv, T, d, causal != 0, softmax_scale, bf16, out32,
                         workspace, s, max_seqlen, cu_seqlens) != hipSuccess)
    return ATTN_ERR_HIP;
  return ATTN_OK;
}

// Shapes of the split-KV forward: the rows sharing one K/V head (Hq / Hkv heads x Nq rows) are
// taken in groups of 32; the grid (batch x K/V head x split x row group) must fit 32 bits.
static int check_splitkv(int B, int Hq, int Hkv, int Nq, int Nk, int d, int num_splits) {
  if (Nq < 1 || Nk < 1 || num_splits < 0) return ATTN_ERR_INVALID;
  const int st = check_sizes(B, Hq, Hkv, Nk, d);
  if (st != ATTN_OK) return st;
  if (Nq > Nk) return ATTN_ERR_INVALID;
  if ((double)B * Hq * Nq * d > 9.0e15) return ATTN_ERR_INVALID;
  const double row_groups = ((double)(Hq / Hkv) * Nq + 31.0) / 32.0;
  if ((double)B * Hkv * row_groups * ((Nk + 127) / 128) > 2.0e9) return ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

size_t attn_fwd_splitkv_workspace_size(int B, int Hq, int Hkv, int Nq, int Nk, int d, int num_splits) {
  if (check_splitkv(B, Hq, Hkv, Nq, Nk, d, num_splits) != ATTN_OK) return 0;
  return eao::splitkv_workspace_bytes(B, Hq, Hkv, Nq, Nk, d, num_splits);
}

int attn_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv,
                     int Nq, int Nk, int d, int causal, float softmax_scale, int dtype, int num_splits,
                     void* workspace, size_t workspace_bytes, attn_stream_t stream) {
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse)) return ATTN_ERR_INVALID;
  if (!scale_ok(softmax_scale)) return ATTN_ERR_INVALID;
  if (dtype != ATTN_F16 && dtype != ATTN_BF16) return dtype == ATTN_FP8_E4M3 ? ATTN_ERR_UNSUPPORTED : ATTN_ERR_INVALID;
  const int st = check_splitkv(B, Hq, Hkv, Nq, Nk, d, num_splits);
  if (st != ATTN_OK) return st;
  if (workspace == nullptr || ((uintptr_t)workspace & 255u) != 0) return ATTN_ERR_WORKSPACE;
  if (workspace_bytes < eao::splitkv_workspace_bytes(B, Hq, Hkv, Nq, Nk, d, num_splits)) return ATTN_ERR_WORKSPACE;
  return eao::launch_fwd_splitkv(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, causal != 0, softmax_scale,
                                 dtype == ATTN_BF16, num_splits, workspace, (hipStream_t)stream) == hipSuccess
             ? ATTN_OK : ATTN_ERR_HIP;
}

int attn_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
                             int Hkv, int Nq, int Nk, int d, int causal, float softmax_scale, int dtype,
                             int num_splits, attn_stream_t stream) {
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse)) return ATTN_ERR_INVALID;
  if (!scale_ok(softmax_scale)) return ATTN_ERR_INVALID;
  if (dtype != ATTN_F16 && dtype != ATTN_BF16) return dtype == ATTN_FP8_E4M3 ? ATTN_ERR_UNSUPPORTED : ATTN_ERR_INVALID;
  const int st = check_splitkv(B, Hq, Hkv, Nq, Nk, d, num_splits);
  if (st != ATTN_OK) return st;
  if (eao::splitkv_workspace_bytes(B, Hq, Hkv, Nq, Nk, d, num_splits) > eao::splitkv_scratch_bytes())
    return ATTN_ERR_SCRATCH;
  // the scratch address is per device: the stream must run on the current device
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return ATTN_ERR_HIP;
  if (stream != nullptr) {
    hipDevice_t sdev = -1;
    if (hipStreamGetDevice((hipStream_t)stream, &sdev) != hipSuccess) return ATTN_ERR_HIP;
    if ((int)sdev != cur) return ATTN_ERR_INVALID;
  }
  void* ws = nullptr;
  if (eao::splitkv_scratch_address(&ws) != hipSuccess) return ATTN_ERR_HIP;
  return eao::launch_fwd_splitkv(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, causal != 0, softmax_scale,
                                 dtype == ATTN_BF16, num_splits, ws, (hipStream_t)stream) == hipSuccess
             ? ATTN_OK : ATTN_ERR_HIP;
}

int attn_clock_probe(unsigned long long* out, int groups, long long ticks, attn_stream_t stream) {
  if (out == nullptr || ((uintptr_t)out & 15u) != 0) return ATTN_ERR_INVALID;
  if (groups < 1 || groups > 1024 || ticks < 1 || ticks > 1000000000LL) return ATTN_ERR_INVALID;
  return eao::launch_clock_probe(out, groups, ticks, (hipStream_t)stream) == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

int attn_mfma_probe(const void* data, long long n, float* out, int groups, int iters, int dtype,
                    attn_stream_t stream) {
  if (dtype != ATTN_BF16 && dtype != ATTN_FP8_E4M3) return ATTN_ERR_UNSUPPORTED;
  if (!aligned16(data) || !aligned16(out)) return ATTN_ERR_INVALID;
  const bool fp8 = dtype == ATTN_FP8_E4M3;
  const long long unit = fp8 ? 32 : 8;          // values per operand fragment of one lane
  if (n < 8192 || n % unit != 0 || groups < 1 || groups > 65536 || iters < 1 || iters > (1 << 20))
    return ATTN_ERR_INVALID;
  const hipError_t e = eao::launch_mfma_probe(data, (size_t)n, fp8, out, groups, iters, (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

int attn_hbm_probe(const void* data, long long bytes, unsigned* out, int groups, attn_stream_t stream) {
  if (!aligned16(data) || !aligned16(out)) return ATTN_ERR_INVALID;
  if (groups < 1 || groups > 65536 || bytes <= 0 || bytes % ((long long)groups * 16384) != 0) return ATTN_ERR_INVALID;
  const long long share = bytes / groups;
  if (share > (1LL << 31)) return ATTN_ERR_INVALID;
  const hipError_t e = eao::launch_hbm_probe((const uint8_t*)data, (uint32_t)share, out, groups, (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

int attn_fp8_prep(const float* x, uint8_t* x_fp8, float* descale, const int8_t* signs, int B, int H, int N, int d,
                  int pow2_scale, attn_stream_t stream) {
  if (!aligned16(x) || !aligned16(x_fp8) || !aligned16(descale)) return ATTN_ERR_INVALID;
  if (signs != nullptr && ((uintptr_t)signs & 15u) != 0) return ATTN_ERR_INVALID;
  const int st = check_sizes(B, H, H, N, d);
  if (st != ATTN_OK) return st;
  const hipError_t e = eao::launch_fp8_prep(x, x_fp8, descale, signs, B, H, N, d, pow2_scale != 0, (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

}  // extern "C"
