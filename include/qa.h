/*
 * qa.h -- C ABI of libqa, causal grouped-query attention over a preallocated
 * KV cache on AMD Instinct MI355X (gfx950).
 *
 * The library computes, for each token of a batch of token sequences:
 *   k' = RoPE(RMSNorm(k)),  q' = RoPE(RMSNorm(q))      (per head, head_dim 128)
 *   cache K[b, g, pos] = bf16(k'),  cache V[b, g, pos] = v
 *   out[t, h] = sum_{j <= pos} softmax_j(scale * q'[t,h] . K[b, h/G, j]) V[b, h/G, j]
 * for three shapes of call: prompt prefill, single-token decode and
 * multi-token verification of a speculative draft block.
 *
 * Sources, cited by page title and section:
 *   "dryft-flash-infer" agent guide, Where the wins are: prefill is a large
 *     share of time; a preallocated, correctly strided KV cache; RMSNorm and
 *     rotary embedding fused; speculative decoding with exact verification.
 *   "dryft-flash-infer" agent guide, Numerics: reductions may be reordered and
 *     accumulated in fp32; the bf16 cast may not move.
 *   "htn.dryft.ai/docs", What to submit: a batch of token sequences, one token
 *     per sequence per step, bf16 Qwen3-4B (32 query heads, 8 KV heads,
 *     head_dim 128).
 *   pegainfer PR #862 (SM120 FlashInfer GDN prefill), review thread: a narrow
 *     C ABI around the kernels that fails validation instead of silently
 *     running another kernel, and launch counters that prove which kernel ran.
 *
 * Conventions for every entry point:
 *   - bf16 tensors are passed as void* to 16-bit storage (bfloat16 bits).
 *   - All tensor pointers are DEVICE pointers and must be 16-byte aligned;
 *     element strides must be multiples of 8.  The caller owns every tensor
 *     and the workspace; the library keeps no pointer after a call returns and
 *     allocates device memory only in qa_cache_alloc when asked to.
 *   - Calls are asynchronous on the given stream (a hipStream_t passed as
 *     void*, NULL = the default stream), perform no host-device
 *     synchronisation and no allocation, and may be captured into a HIP graph.
 *   - Validation is done on the host before any launch.  On failure the call
 *     returns a negative qa_status, launches nothing and records a message for
 *     qa_last_error().  There is no fallback kernel.
 *   - Device-side checks (positions and sequence offsets live in device
 *     memory): a token whose position is outside [0, capacity) (or outside
 *     [0, max_ctx) for decode/verify) is not written to the cache, its output
 *     row is set to zero and a bit is set in the workspace error word (read it
 *     with qa_device_error).  No kernel reads or writes outside the buffers
 *     described by its arguments, whatever the device-side values are.
 *   - Calls that share a workspace must not run concurrently.
 */
#ifndef QA_H
#define QA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  QA_OK = 0,
  QA_ERR_NULL = -1,        /* a required pointer is NULL */
  QA_ERR_SHAPE = -2,       /* inconsistent or out-of-range sizes */
  QA_ERR_UNSUPPORTED = -3, /* head_dim != 128 or GQA group not in {1,2,4,8} */
  QA_ERR_ALIGN = -4,       /* pointer or stride misaligned */
  QA_ERR_CAPACITY = -5,    /* context longer than the cache */
  QA_ERR_WORKSPACE = -6,   /* workspace missing or too small */
  QA_ERR_HIP = -7,         /* a HIP runtime call failed */
  QA_ERR_DEVICE = -8       /* debug mode only: a kernel of this call set a
                              QA_DEVERR_* bit in the workspace error word */
} qa_status;

/* Operation codes for qa_workspace_bytes. */
enum { QA_OP_PREFILL = 0, QA_OP_DECODE = 1, QA_OP_VERIFY = 2 };

/* Device-side error bits (qa_device_error). */
enum {
  QA_DEVERR_POSITION = 1, /* a position outside the cache or the context */
  QA_DEVERR_SEQLENS = 2,  /* cu_seqlens not increasing from 0 to total_tokens,
                             or a sequence longer than max_seqlen */
  QA_DEVERR_MERGE = 4     /* decode: the split workgroups of a (sequence, kv
                             head) did not all run on one XCD, so their partials
                             were not merged inside the launch; that pair's
                             rows are zeroed */
};

/*
 * KV cache descriptor.  K and V are bf16 arrays indexed
 *   [b * stride_b + g * stride_h + slot * stride_pos + i],  i < head_dim,
 * one row per sequence b < batch, one slot per absolute position
 * ("dryft-flash-infer" agent guide, Where the wins are: preallocated,
 * correctly strided cache).  The cache holds post-RoPE K and raw V.
 */
typedef struct qa_cache {
  void* k;
  void* v;
  int32_t batch;
  int32_t n_kv_heads;
  int32_t capacity;
  int32_t head_dim;
  int64_t stride_b;   /* elements */
  int64_t stride_h;   /* elements */
  int64_t stride_pos; /* elements */
  int32_t owns;       /* 1 if qa_cache_alloc allocated k and v */
} qa_cache;

/*
 * Per-call model parameters.  softmax_scale multiplies q'.k (1/sqrt(128) for
 * Qwen3); rope_theta is the rotary base (1e6 for Qwen3-4B); rms_eps is the
 * epsilon inside the RMSNorm square root.  q_norm_w / k_norm_w are bf16
 * [head_dim] device arrays of RMSNorm weights, or NULL for all ones.
 */
typedef struct qa_params {
  int32_t n_q_heads;
  float softmax_scale;
  double rope_theta;
  double rms_eps;
  const void* q_norm_w;
  const void* k_norm_w;
} qa_params;

/*
 * Fill a cache descriptor with dense strides
 * (stride_pos = head_dim, stride_h = capacity*head_dim, stride_b = n_kv_heads*stride_h).
 * If k_mem and v_mem are both non-NULL they are used as the K and V arrays
 * (owns = 0; the caller keeps ownership).  If both are NULL the library
 * allocates them with hipMalloc (owns = 1) and does not initialise them.
 * Errors: QA_ERR_NULL (out NULL, or exactly one of k_mem/v_mem NULL),
 * QA_ERR_SHAPE, QA_ERR_UNSUPPORTED (head_dim != 128), QA_ERR_ALIGN,
 * QA_ERR_HIP (allocation failed).
 */
qa_status qa_cache_alloc(qa_cache* out, int batch, int n_kv_heads,
                         int capacity, int head_dim, void* k_mem,
                         void* v_mem);

/* Free what qa_cache_alloc allocated (nothing if owns == 0); zero *c. */
qa_status qa_cache_free(qa_cache* c);

/*
 * Bytes of workspace the given operation needs for these sizes (0 on invalid
 * sizes).  max_ctx is the largest context (position + 1) a decode/verify call
 * will see; block_len is the draft length for QA_OP_VERIFY.  For
 * QA_OP_PREFILL pass the call's total token count as max_ctx.
 */
size_t qa_workspace_bytes(int op, int batch, int n_q_heads, int n_kv_heads,
                          int max_ctx, int block_len);

/*
 * Clear a workspace (its device error word, and decode's merge counters) with
 * a fill kernel on stream s.  Run once after allocating a workspace, before
 * its first use.  Split-K partials in the workspace are fully rewritten by
 * every call.
 */
qa_status qa_workspace_init(void* ws, size_t ws_bytes, void* stream);

/*
 * Prompt prefill of a packed batch ("dryft-flash-infer" agent guide, Where the
 * wins are: Prefill).  Sequence i < n_seq owns tokens
 * cu_seqlens[i] .. cu_seqlens[i+1]-1 and cache row i; token t sits at
 * positions[t].  The call first writes K/V of all its tokens to the cache,
 * then every token attends to slots 0 .. positions[t] of its row (earlier
 * slots may come from previous calls: chunked prefill).  Every slot a
 * sequence's queries can see must have been written by this or an earlier
 * call.
 *   q   bf16 [total_tokens][n_q_heads][128],  token stride q_tok_stride
 *   k,v bf16 [total_tokens][n_kv_heads][128], token stride kv_tok_stride
 *   cu_seqlens int32 [n_seq+1] (device), positions int32 [total_tokens] (device)
 *   out bf16 [total_tokens][n_q_heads][128] (dense)
 *   lse fp32 [total_tokens][n_q_heads] natural-log log-sum-exp, or NULL
 *   max_seqlen >= every sequence length (sizes the launch grid)
 *   ws  workspace of qa_workspace_bytes(QA_OP_PREFILL, ..., total_tokens, 0)
 *       bytes: the error word and the queries' cos/sin table (8 bytes per
 *       token and rotation pair), written and read within the call
 * total_tokens == 0 is a valid no-op.
 */
qa_status qa_prefill(const qa_cache* c, const qa_params* p, const void* q,
                     const void* k, const void* v, int64_t q_tok_stride,
                     int64_t kv_tok_stride, const int32_t* cu_seqlens,
                     const int32_t* positions, int n_seq, int total_tokens,
                     int max_seqlen, void* out, float* lse, void* ws,
                     size_t ws_bytes, void* stream);

/*
 * One cached decode step ("dryft-flash-infer" agent guide, Invariants: one
 * token per sequence per step; Where the wins are: per-step overhead).  The
 * new token of sequence b < batch sits at positions[b]; its K/V are written
 * to that slot, then it attends to slots 0 .. positions[b].
 *   q bf16 [batch][n_q_heads][128], k,v bf16 [batch][n_kv_heads][128] (dense)
 *   positions int32 [batch] (device); every positions[b] < max_ctx <= capacity
 *   out bf16 [batch][n_q_heads][128], lse fp32 [batch][n_q_heads] or NULL
 * The launch grid depends only on (batch, heads, max_ctx), so a captured graph
 * stays valid while positions advance in device memory.
 *   ws  workspace of qa_workspace_bytes(QA_OP_DECODE, batch, ..., max_ctx, 0)
 *       bytes.  When batch * n_kv_heads is a multiple of 8 the split-K
 *       partials are merged inside the one launch, through one counter per
 *       (sequence, kv head) kept in the workspace.  The counters must be zero
 *       when a call starts, and every call returns them to zero.  So clear
 *       the workspace with qa_workspace_init before the first decode call, and
 *       again after the buffer served anything else (another operation, or
 *       decode with other batch, heads or max_ctx).  Calls sharing a
 *       workspace must be ordered on one stream.
 */
qa_status qa_decode(const qa_cache* c, const qa_params* p, const void* q,
                    const void* k, const void* v, const int32_t* positions,
                    int batch, int max_ctx, void* out, float* lse, void* ws,
                    size_t ws_bytes, void* stream);

/*
 * qa_decode without a workspace, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Same arguments, kernels and results as qa_decode, except
 * that the split-K partials and the in-launch merge counters live in a
 * library-held device array of 16 MiB per GPU (held until the process ends),
 * and device-side errors (QA_DEVERR_* bits) are OR-ed into *dev_err, a
 * caller-owned device int32 (NULL: not reported).  Sizes whose decode
 * workspace (qa_workspace_bytes(QA_OP_DECODE, ...)) exceeds 16 MiB are
 * rejected with QA_ERR_WORKSPACE.  The array is cleared by a fill kernel on
 * `stream` at the first eager call on a device (a call captured before that
 * carries the clear in its graph); every call returns the merge counters to
 * zero.  All calls on one GPU share its array: calls that overlap on one GPU
 * (another stream, another thread) race, so order them on one stream.
 * Allocates nothing: no hipMalloc, hipFree or allocating library call.
 */
qa_status qa_decode_noalloc(const qa_cache* c, const qa_params* p, const void* q,
                            const void* k, const void* v, const int32_t* positions,
                            int batch, int max_ctx, void* out, float* lse,
                            int32_t* dev_err, void* stream);

/*
 * Exact verification of a block_len-token draft per sequence
 * ("dryft-flash-infer" agent guide, Where the wins are: speculative decoding
 * with exact verification).  Draft token i of sequence b sits at
 * start_pos[b] + i; all block_len K/V are written first, then token i attends
 * to slots 0 .. start_pos[b] + i (its own and earlier draft tokens included).
 * Rolling back a rejected suffix is the caller's: it rewinds its own length.
 *   q bf16 [batch][block_len][n_q_heads][128]
 *   k,v bf16 [batch][block_len][n_kv_heads][128] (dense)
 *   start_pos int32 [batch] (device); start_pos[b] + block_len <= max_ctx
 *   out bf16 [batch][block_len][n_q_heads][128], lse fp32 [..][n_q_heads] or NULL
 * Requires block_len * (n_q_heads / n_kv_heads) <= 128.
 */
qa_status qa_verify(const qa_cache* c, const qa_params* p, const void* q,
                    const void* k, const void* v, const int32_t* start_pos,
                    int batch, int block_len, int max_ctx, void* out,
                    float* lse, void* ws, size_t ws_bytes, void* stream);

/*
 * Hidden-state RMSNorm with the residual add, in the reference model's cast
 * placement ("dryft-flash-infer" agent guide, Where the wins are: RMSNorm is
 * small, repeated and safe to fuse; Numerics: reductions may be reordered, the
 * bf16 cast may not move).  For each of n_tokens rows of `hidden` values:
 *   r   = bf16(x + residual)               (r = x when residual is NULL)
 *   out = bf16(weight * bf16(r / sqrt(mean(r^2) + eps)))   (weight NULL = 1)
 * and residual, when given, is overwritten with r (the updated residual
 * stream).  Every step other than the three bf16 roundings is exact up to the
 * order of the sum of squares.
 *   x, residual, out bf16 [n_tokens][hidden] (dense), weight bf16 [hidden]
 *   hidden a multiple of 8, at most 8192; out may not alias x or residual
 * n_tokens == 0 is a valid no-op (the pointers may then be NULL).
 * Asynchronous on `stream`, allocates nothing.
 */
qa_status qa_rmsnorm_hidden(const void* x, void* residual, const void* weight,
                            int n_tokens, int hidden, double eps, void* out,
                            void* stream);

/*
 * The attention epilogue of one decoder layer in the reference model's cast
 * placement ("dryft-flash-infer" agent guide, Where the wins are: RMSNorm and
 * the attention epilogue are small and safe to fuse; Numerics: sums may be
 * reordered and accumulated in fp32, the bf16 casts may not move).  For each
 * of n_tokens rows:
 *   h        = bf16(o . w_o^T)              (output projection, fp32 sums)
 *   residual = bf16(residual + h)           (updated in place)
 *   out      = bf16(norm_w * bf16(residual / sqrt(mean(residual^2) + eps)))
 * The last line is qa_rmsnorm_hidden's arithmetic on the new residual.
 *   o        bf16 [n_tokens][in_dim], token stride o_tok_stride (elements;
 *            the attention output with its heads concatenated, e.g. the
 *            [T][n_q_heads][128] output of qa_prefill with in_dim = n_q_heads*128)
 *   w_o      bf16 [hidden][in_dim]: the linear layer's weight, one row per
 *            output feature
 *   residual bf16 [n_tokens][hidden] (dense), read and overwritten
 *   norm_w   bf16 [hidden] post-attention norm weight, or NULL for ones
 *   out      bf16 [n_tokens][hidden] (dense), may not alias residual
 * Requires in_dim a multiple of 64, hidden a multiple of 128 and at most
 * 8192.  Two kernels (the projection GEMM, then the norm), asynchronous on
 * `stream`, no allocation.  n_tokens == 0 is a valid no-op.
 */
qa_status qa_attn_epilogue(const void* o, int64_t o_tok_stride, const void* w_o,
                           void* residual, const void* norm_w, int n_tokens, int in_dim,
                           int hidden, double eps, void* out, void* stream);

/* Plain device copy of `bytes` (multiple of 16) from src to dst on `stream`;
 * the calibration kernel for bandwidth and traffic measurements. */
qa_status qa_copy(const void* src, void* dst, size_t bytes, void* stream);

/* Name of a status code. */
const char* qa_status_str(qa_status s);

/* Detail of the last failure on the calling thread ("" if none). */
const char* qa_last_error(void);

/*
 * Process-wide counters: [0] prefill launches, [1] decode launches,
 * [2] verify launches, [3] kernels launched, [4] calls rejected by
 * validation, [5] HIP launch failures, [6] workspace inits, [7] copies.
 */
void qa_get_counters(uint64_t out[8]);
void qa_reset_counters(void);

/*
 * Synchronise `stream`, then read and clear the device error word of `ws`
 * into *code (a mask of QA_DEVERR_* bits, 0 if none).  Not for use inside a
 * captured graph.
 */
qa_status qa_device_error(void* ws, void* stream, int32_t* code);

/*
 * Debug mode, for bringing up a caller (fail-closed checking: pegainfer PR
 * #862, review thread).  When on, every call that launches kernels then
 * synchronises its stream and returns QA_ERR_HIP if a HIP error is pending,
 * or QA_ERR_DEVICE if its workspace error word (decode_noalloc: *dev_err)
 * holds any QA_DEVERR_* bit; the word is left as it is.  Calls on a stream
 * that is being captured into a graph skip the check.  Off by default; the
 * environment variable QA_DEBUG=1 turns it on for the process (read at the
 * first call), qa_set_debug(1) or (0) at any time.  Debug mode costs a host
 * synchronisation per call.
 */
void qa_set_debug(int on);

#ifdef __cplusplus
}
#endif

#endif /* QA_H */
