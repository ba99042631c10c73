/*
 * attn.h -- C ABI of the MI355X (gfx950) exact-attention library (libattn.so).
 *
 * Exact scaled-dot-product attention O = softmax(scale * Q K^T) V, computed by fused tiled
 * kernels with an online softmax: the N x N score matrix never reaches HBM, each query row
 * keeps a running maximum and running sum, the output is divided by the sum once at the end,
 * and the per-row logsumexp is saved for the backward pass, which recomputes the scores and
 * probabilities from Q, K, V and that logsumexp.
 *   - "FlashAttention (NeurIPS 2022)" study notes, sections "Online Softmax", "FlashAttention"
 *     and "Backward - Recomputation";
 *   - "FlashAttention-2: Faster Attention with Better Parallelism and Work Partitioning",
 *     OpenReview discussion: unnormalised accumulator with one final division, logsumexp saved
 *     instead of max and sum, causal key blocks after the query skipped, parallelism over
 *     batch x head x query block, grouped-query attention (several query heads per K/V head);
 *   - "FlashAttention-3: Fast and Accurate Attention with Asynchrony and Low-precision",
 *     abstract: FP8 with block quantisation and incoherent processing.
 *
 * Conventions shared by every entry point
 *   Pointers     device pointers (hipMalloc'd or equivalent), 16-byte aligned, owned by the
 *                caller.  The library never allocates, frees or synchronises, holds no global
 *                mutable state, and is safe to call from several host threads.
 *   Layout       row-major contiguous [B, H, N, d]: Q, O, dO, dQ have H = Hq heads; K, V, dK,
 *                dV have H = Hkv heads.  Query head h reads K/V head h / (Hq / Hkv).
 *                LSE is float [B, Hq, N], natural logarithm.
 *   Sizes        B, Hq, Hkv, N >= 1; Hq % Hkv == 0; d in {64, 128}; query and key lengths are
 *                both N.  causal != 0 lets query i see keys j <= i only.
 *   Scale        softmax_scale must be finite and > 0 (the usual value is 1 / sqrt(d)).
 *   Streams      stream is a hipStream_t (NULL = the default stream).  Every call only enqueues
 *                work on that stream and returns; outputs are valid after the stream reaches
 *                that point.  Outputs are overwritten, never accumulated into.
 *   Errors       arguments are checked on the host before anything is enqueued; a failed check
 *                returns a nonzero attn_status_t and enqueues nothing.  A launch failure
 *                reported by the HIP runtime returns ATTN_ERR_HIP.  Faults inside a kernel show
 *                up at the caller's next synchronisation.  NaN/Inf inputs propagate.
 */
#ifndef EXACT_ATTENTION_ONLINE_ATTN_H
#define EXACT_ATTENTION_ONLINE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void* attn_stream_t; /* a hipStream_t */

typedef enum {
  ATTN_F16 = 0,       /* IEEE binary16 storage */
  ATTN_BF16 = 1,      /* bfloat16 storage */
  ATTN_FP8_E4M3 = 2,  /* OCP FP8 E4M3 (e4m3fn) storage with per-block float scales */
  ATTN_F32 = 3        /* IEEE binary32: only as the gradient dtype of a backward call */
} attn_dtype_t;

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_INVALID = 1,     /* null/misaligned pointer, bad size, bad scale, bad dtype */
  ATTN_ERR_UNSUPPORTED = 2, /* well-formed but not built: head dim other than 64/128, ... */
  ATTN_ERR_WORKSPACE = 3,   /* workspace missing or smaller than attn_bwd_workspace_size() */
  ATTN_ERR_HIP = 4,         /* the HIP runtime rejected a launch */
  ATTN_ERR_SCRATCH = 5      /* larger than the static scratch of attn_fwd_splitkv_noalloc */
} attn_status_t;

/* Forward pass.
 *   q [B,Hq,N,d], k, v [B,Hkv,N,d] in `dtype`; o [B,Hq,N,d] in `dtype` (bfloat16 when dtype is
 *   ATTN_FP8_E4M3); lse [B,Hq,N] float, natural log: lse = m + ln(sum_j exp(s_j - m)).
 *   ATTN_FP8_E4M3 only: q_descale, k_descale, v_descale are float [B,H,ceil(N/128)] (H = Hq for
 *   q, Hkv for k and v): the value of a stored code x in rows 128*i .. 128*i+127 of a head is
 *   e4m3(x) * descale[i].  They must be NULL for ATTN_F16 / ATTN_BF16.
 *   ATTN_F16 / ATTN_BF16 results are deterministic, and a head's o and lse are bit-identical
 *   whatever the other heads and batch entries of the call are (the query-block size picked
 *   from the grid size does not change a row's arithmetic).
 * Returns an attn_status_t. */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int B, int Hq, int Hkv, int N, int d, int causal, float softmax_scale, int dtype,
             const float* q_descale, const float* k_descale, const float* v_descale,
             attn_stream_t stream);

/* Forward with a local (sliding-window) mask and/or an ALiBi bias ("FlashAttention-2: Faster
 * Attention with Better Parallelism and Work Partitioning", OpenReview discussion, author
 * responses: FA2 supports ALiBi, and local, i.e. sliding-window, attention).  Arguments as for
 * attn_fwd (dtype ATTN_F16 or ATTN_BF16), plus:
 *   window: 0 = no window; otherwise key j is visible to query i only if i - j < window, and,
 *     when causal is 0, also j - i < window (with causal, j <= i as well).
 *   alibi_slopes: NULL, or device float [Hq] (4-byte aligned): score (i, j) of query head h is
 *     softmax_scale * q_i . k_j - alibi_slopes[h] * |i - j|.
 * With window 0 and no slopes the result equals attn_fwd's.  Returns an attn_status_t. */
int attn_fwd_ext(const void* q, const void* k, const void* v, void* o, float* lse,
                 int B, int Hq, int Hkv, int N, int d, int causal, float softmax_scale, int dtype,
                 int window, const float* alibi_slopes, attn_stream_t stream);

/* Forward over variable-length sequences packed without padding ("FlashAttention-2: Faster
 * Attention with Better Parallelism and Work Partitioning", OpenReview discussion, author
 * responses: sequences are concatenated with no padding token and an array gives the lengths).
 *   q [Hq,T,d], k, v [Hkv,T,d], o [Hq,T,d] in `dtype` (ATTN_F16 / ATTN_BF16), lse [Hq,T] float:
 *   the [B,H,N,d] layout of attn_fwd with the B sequences concatenated along the rows.
 *   cu_seqlens: device int32 [B+1], 0 = cu_seqlens[0] <= ... <= cu_seqlens[B] = T; sequence b is
 *   rows cu_seqlens[b] .. cu_seqlens[b+1]-1 and attends only within itself (causal: as in
 *   attn_fwd, per sequence).  Entries are read on the device and clamped to [0, T], so malformed
 *   offsets give wrong rows, never an access outside the tensors.
 *   max_seqlen: at least the longest sequence (1 <= max_seqlen <= T); rows past max_seqlen of a
 *   longer sequence are not computed.  Sequences of length 0 are allowed.
 * Returns an attn_status_t. */
int attn_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                    const int* cu_seqlens, int B, int Hq, int Hkv, int T, int max_seqlen, int d,
                    int causal, float softmax_scale, int dtype, attn_stream_t stream);

/* Backward of attn_fwd_ext: gradients of L = <O, dO> with the sliding window and/or ALiBi bias
 * of attn_fwd_ext ("FlashAttention-2: Faster Attention with Better Parallelism and Work
 * Partitioning", OpenReview discussion, author responses: ALiBi and local attention;
 * "FlashAttention (NeurIPS 2022)" notes, "Backward - Recomputation").  The bias does not depend
 * on q or k, so the gradients keep the form of attn_bwd with P recomputed under the same mask
 * and bias.  Arguments as for attn_bwd (same workspace size, attn_bwd_workspace_size, and the
 * same grad_dtype choice), with o and lse from attn_fwd_ext and the same causal flag, scale,
 * window and alibi_slopes.
 * window 0 and NULL slopes give exactly attn_bwd's gradients up to rounding order.
 * Returns an attn_status_t. */
int attn_bwd_ext(const void* q, const void* k, const void* v, const void* o, const void* dout,
                 const float* lse, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int N,
                 int d, int causal, float softmax_scale, int dtype, int grad_dtype, int window,
                 const float* alibi_slopes, void* workspace, size_t workspace_bytes,
                 attn_stream_t stream);

/* Backward of attn_fwd_varlen: gradients of L = <O, dO> for variable-length sequences packed
 * without padding ("FlashAttention-2: Faster Attention with Better Parallelism and Work
 * Partitioning", OpenReview discussion, author responses: concatenated sequences and an array of
 * lengths; "FlashAttention (NeurIPS 2022)" notes, "Backward - Recomputation").  Each sequence's
 * gradients are those attn_bwd gives for that sequence alone (dq bit for bit; dk and dv up to the
 * order of their fp32 additions, since attn_bwd splits the dK/dV phase of small grouped problems
 * and this entry point never does).
 *   q, o, dout [Hq,T,d], k, v [Hkv,T,d] in `dtype` (ATTN_F16 / ATTN_BF16), lse [Hq,T] float from
 *   attn_fwd_varlen with the same cu_seqlens, causal flag and scale; cu_seqlens, B, T and
 *   max_seqlen as for attn_fwd_varlen.  Outputs dq [Hq,T,d], dk, dv [Hkv,T,d] in `grad_dtype`
 *   (`dtype` or ATTN_F32, as for attn_bwd), dk and dv summed over the query heads that share each
 *   K/V head; rows that belong to no sequence (past cu_seqlens[B]) are not written.
 *   workspace: device memory of at least attn_bwd_varlen_workspace_size() bytes, 256-byte
 *   aligned, owned by the caller; clobbered.  A sequence longer than max_seqlen (rounded up to
 *   64) gets unspecified gradients but no access outside the buffers.
 * Returns an attn_status_t. */
size_t attn_bwd_varlen_workspace_size(int B, int Hq, int Hkv, int max_seqlen, int d);
int attn_bwd_varlen(const void* q, const void* k, const void* v, const void* o, const void* dout,
                    const float* lse, void* dq, void* dk, void* dv, const int* cu_seqlens, int B,
                    int Hq, int Hkv, int T, int max_seqlen, int d, int causal, float softmax_scale,
                    int dtype, int grad_dtype, void* workspace, size_t workspace_bytes,
                    attn_stream_t stream);

/* Bytes of device workspace attn_bwd needs, linear in N (no N x N buffer); with Npad = N rounded
 * up to a multiple of 64: -D = -rowsum(dO * O) and LSE * log2(e) as float [B,Hq,Npad] each,
 * i.e. 2 * roundup(4 * B * Hq * Npad, 256) bytes.  Grouped-query problems (Hq > Hkv) whose B * Hkv * ceil(N / 128) is below 256 split the
 * dK/dV phase S = min(ceil(512 / (B * Hkv * ceil(N / 128))), 2 * Hq / Hkv) ways, so that it fills
 * the GPU, and add S * 2 * B * Hkv * N * d * 4 bytes for the float shares (added in a fixed
 * order, so the gradients stay deterministic).  0 if the sizes are invalid. */
size_t attn_bwd_workspace_size(int B, int Hq, int Hkv, int N, int d);

/* Backward pass of L = <O, dO> ("FlashAttention (NeurIPS 2022)" notes, "Backward -
 * Recomputation"; dV = P^T dO from the FlashAttention-2 discussion).
 *   q, k, v, o, dout, lse as produced by/for attn_fwd with the same sizes, causal flag and
 *   scale; dtype ATTN_F16 or ATTN_BF16.  Outputs dq [B,Hq,N,d] and dk, dv [B,Hkv,N,d] in
 *   `grad_dtype`; dk and dv are summed over the query heads that share each K/V head.
 *   grad_dtype: `dtype` (the fp32 accumulators rounded to nearest even) or ATTN_F32 (the
 *   accumulators themselves, 4 bytes per element).  Anything else is ATTN_ERR_INVALID.  A group
 *   sum of several query heads can exceed 8 in magnitude, where half a bfloat16 step (2^-5) is
 *   already more than an absolute error bound of 3e-2; ATTN_F32 keeps such sums free of that
 *   rounding.
 *   workspace: device memory of at least attn_bwd_workspace_size() bytes, 256-byte aligned,
 *   owned by the caller; its contents on entry do not matter and are clobbered.
 *   No atomics: results are deterministic, and a head's dq is bit-identical whatever the other
 *   heads and batch entries of the call are.
 * Returns an attn_status_t. */
int attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
             const float* lse, void* dq, void* dk, void* dv,
             int B, int Hq, int Hkv, int N, int d, int causal, float softmax_scale, int dtype,
             int grad_dtype, void* workspace, size_t workspace_bytes, attn_stream_t stream);

/* The three phases attn_bwd runs, for callers that schedule or time them separately.  With the
 * same arguments and workspace, preprocess followed by dkdv and dq (in either order, or on two
 * streams once preprocess is complete) produces exactly what attn_bwd produces; attn_bwd is
 * these three calls on one stream.
 *   attn_bwd_preprocess: -D = -rowsum(dO * O) and LSE * log2(e) into the workspace (q and k
 *                        are checked like the other pointers but not read).
 *   attn_bwd_dkdv:       dK, dV written (the probabilities are recomputed from q, k and lse).
 *   attn_bwd_dq:         dQ written (the probabilities are recomputed from q, k and lse).
 * Arguments mean what they mean for attn_bwd (preprocess takes no grad_dtype: it writes only
 * the workspace); each returns an attn_status_t. */
int attn_bwd_preprocess(const void* q, const void* k, const void* o, const void* dout,
                        const float* lse, int B, int Hq, int Hkv, int N, int d, int dtype,
                        void* workspace, size_t workspace_bytes, attn_stream_t stream);
int attn_bwd_dkdv(const void* q, const void* k, const void* v, const void* dout, const float* lse,
                  void* dk, void* dv, int B, int Hq, int Hkv, int N, int d, int causal,
                  float softmax_scale, int dtype, int grad_dtype, const void* workspace,
                  size_t workspace_bytes, attn_stream_t stream);
int attn_bwd_dq(const void* q, const void* k, const void* v, const void* dout, const float* lse,
                void* dq, int B, int Hq, int Hkv, int N, int d, int causal, float softmax_scale,
                int dtype, int grad_dtype, const void* workspace, size_t workspace_bytes,
                attn_stream_t stream);

/* Split-KV forward for decoding ("FlashAttention-2: Faster Attention with Better Parallelism and
 * Work Partitioning", OpenReview discussion: the author response on decoding and the review
 * summary on splitting the KV cache among thread blocks to saturate memory bandwidth): few query
 * rows per head against a long key/value sequence.  The keys of each (batch, K/V head) are cut
 * into splits processed by separate workgroups; each split's exact partial result and logsumexp
 * are combined by LSE = ln sum_s exp(LSE_s), O = sum_s exp(LSE_s - LSE) O_s.
 *   q [B,Hq,Nq,d]; k, v [B,Hkv,Nk,d]; o [B,Hq,Nq,d] in `dtype` (ATTN_F16 / ATTN_BF16);
 *   lse [B,Hq,Nq] float, natural log.  Requires 1 <= Nq <= Nk, else ATTN_ERR_INVALID.  The
 *   (Hq/Hkv) * Nq rows that share a K/V head are processed 32 at a time (workgroups of one key
 *   split and K/V head differ only in their group of 32 rows), so up to 32 rows per K/V head
 *   stream the keys once and more rows re-read them mostly from the L2 cache.
 *   causal: query i sits at position Nk - Nq + i and sees keys j <= Nk - Nq + i (with Nq = 1
 *   every key is visible).
 *   num_splits: splits per (batch, K/V head), 0 = chosen for about two workgroups per compute
 *   unit with splits of at least 512 keys; clamped to the number of 128-key tiles.
 *   workspace: device memory of at least attn_fwd_splitkv_workspace_size() bytes (the float
 *   partial outputs and logsumexps of every split), 256-byte aligned, owned by the caller.
 * Returns an attn_status_t. */
size_t attn_fwd_splitkv_workspace_size(int B, int Hq, int Hkv, int Nq, int Nk, int d, int num_splits);
int attn_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                     int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal, float softmax_scale,
                     int dtype, int num_splits, void* workspace, size_t workspace_bytes,
                     attn_stream_t stream);

/* attn_fwd_splitkv without a workspace argument, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * Arguments and results as for attn_fwd_splitkv (same kernels, same split plan, so the same
 * outputs bit for bit).  The split partials go to a static device buffer of
 * ATTN_SPLITKV_SCRATCH_BYTES (8 MiB) per GPU that the library holds until the process ends; the
 * call allocates nothing.  A problem whose attn_fwd_splitkv_workspace_size exceeds the buffer
 * returns ATTN_ERR_SCRATCH and enqueues nothing.  The stream must belong to the current device
 * (else ATTN_ERR_INVALID).  Every call on one GPU shares that GPU's buffer, which keeps the last
 * call's contents (nothing in it needs clearing: each call writes every partial it reads), so
 * calls that overlap on one GPU -- on different streams or from different threads -- race and
 * must be serialised by the caller.  Returns an attn_status_t. */
#define ATTN_SPLITKV_SCRATCH_BYTES ((size_t)8 << 20)
int attn_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                             int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal,
                             float softmax_scale, int dtype, int num_splits, attn_stream_t stream);

/* FP8 preparation ("FlashAttention-3 ...", abstract: block quantisation and incoherent
 * processing).  x float [B,H,N,d]; when signs (int8 [d], entries +1/-1) is not NULL each row is
 * first replaced by (row * signs) H_d / sqrt(d), H_d the Sylvester Hadamard matrix, computed in
 * float32 with the butterfly stages in order h = 1, 2, ..., d/2.  Then for every block of 128
 * rows of a head: scale = amax / 448 (1 if amax == 0), or with pow2_scale != 0 the smallest power
 * of two p with 448 p >= amax (1 if amax == 0); codes = e4m3(x / scale) rounded to nearest even
 * and saturated to +-448.  Writes x_fp8 uint8 [B,H,N,d] and descale float [B,H,ceil(N/128)]
 * (= scale).  attn_fwd applies power-of-two V scales exactly inside its matrix multiplies (the
 * E8M0 block-scale operand of gfx950's fp8 MFMA), any other V scale by rescaling its
 * accumulator; Q and K scales of either kind cost nothing extra.  Returns an attn_status_t. */
int attn_fp8_prep(const float* x, uint8_t* x_fp8, float* descale, const int8_t* signs,
                  int B, int H, int N, int d, int pow2_scale, attn_stream_t stream);

/* Measurement aid, not a step of the attention method: the engine clock a workload ran at.
 * Launches `groups` single-wave workgroups on `stream`; each reads the shader clock counter
 * (one tick per engine clock) and the 100 MHz real-time counter, sleeps until `ticks` real-time
 * ticks have passed, and writes out[2 i] = engine clocks elapsed, out[2 i + 1] = real-time ticks
 * elapsed (uint64, device memory, 16-byte aligned).  Workgroup i starts on XCD i % 8 of an MI355X,
 * so 8 groups sample every XCD; its clock is 100 MHz * out[2 i] / out[2 i + 1].  Launched on a
 * second stream beside a workload it samples the clock that workload runs at; its waves mostly
 * sleep but each holds a wave slot on one compute unit.  1 <= groups <= 1024 and
 * 1 <= ticks <= 10^9 (10 s), else ATTN_ERR_INVALID.  Returns an attn_status_t. */
int attn_clock_probe(unsigned long long* out, int groups, long long ticks, attn_stream_t stream);

/* Measurement aid, not a step of the attention method: the dense bf16 or fp8 matrix-core rate on
 * given operand data.  The matrix cores draw power according to the bits they multiply and the
 * engine clock follows the board's power limit, so the attainable rate depends on the data: this
 * bounds what any kernel of that type can reach on such inputs.  Launches `groups` workgroups of
 * 512 threads (8 waves: two per SIMD of a compute unit); each wave loads 8 A and 8 B operand
 * fragments from `data` (n values, device memory, read only; positions taken modulo n) and
 * issues iters x 32 back-to-back MFMAs into four fp32 accumulators: dtype ATTN_BF16, n bfloat16
 * values, 16-byte fragments, v_mfma_f32_32x32x16_bf16 (32768 flops each); dtype ATTN_FP8_E4M3,
 * n e4m3 codes, 32-byte fragments, v_mfma_scale_f32_32x32x64_f8f6f4 with unit scales (131072
 * flops each).  Every thread then writes the sum of its accumulators to out[512 * group +
 * thread] (groups * 512 floats, device memory).  The launch does groups * 8 * 32 * iters times
 * the flops of one MFMA.  data and out 16-byte aligned, n >= 8192 and a multiple of 8 (bf16) or
 * 32 (fp8), 1 <= groups <= 65536, 1 <= iters <= 2^20, else ATTN_ERR_INVALID; another dtype,
 * ATTN_ERR_UNSUPPORTED.  Returns an attn_status_t. */
int attn_mfma_probe(const void* data, long long n, float* out, int groups, int iters, int dtype,
                    attn_stream_t stream);

/* Measurement aid, not a step of the attention method: the rate at which the chip streams
 * device memory into LDS with the direct buffer -> LDS loads of the kernels, in the split-KV
 * decoding kernel's pattern, which bounds what a memory-bound kernel of that shape can reach.
 * Launches `groups` workgroups of one wave; workgroup g streams bytes [g * share, (g + 1) * share)
 * of `data` (device memory, read only; share = bytes / groups) in 16 KB stages through a ring of
 * four LDS slots, requesting three stages ahead, and lane l of it writes to out[64 g + l] (groups
 * * 64 unsigned words, device memory) the sum modulo 2^32 of the 32-bit words it loaded, so the
 * sum of out modulo 2^32 is that of every 32-bit word of data.  data and out 16-byte aligned,
 * 1 <= groups <= 65536, bytes > 0 a multiple of groups * 16384, share <= 2^31, else
 * ATTN_ERR_INVALID.  Returns an attn_status_t. */
int attn_hbm_probe(const void* data, long long bytes, unsigned* out, int groups, attn_stream_t stream);

/* Static, human-readable text for a status code. */
const char* attn_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* EXACT_ATTENTION_ONLINE_ATTN_H */
