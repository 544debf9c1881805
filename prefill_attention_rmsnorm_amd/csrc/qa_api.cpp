// Host side of libqa: argument validation, launch, counters, error text.
//
// pegainfer PR #862 (SM120 FlashInfer GDN prefill), review thread: the C ABI
// around the kernels validates ABI and geometry and fails instead of silently
// running another kernel, and counts successful launches so that tests can
// prove which kernel ran.  Every check below runs before any HIP call.
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>

#include "qa.h"
#include "qa_internal.h"
#include "rmsnorm.h"
#include "verify_layout.h"

namespace {

thread_local std::string g_last_error;
std::atomic<uint64_t> g_counters[8];

enum {
  CNT_PREFILL = 0, CNT_DECODE, CNT_VERIFY, CNT_KERNELS, CNT_REJECTED,
  CNT_HIP_FAIL, CNT_WS_INIT, CNT_COPY
};

qa_status fail(qa_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  g_counters[CNT_REJECTED].fetch_add(1);
  return s;
}

qa_status hip_fail(hipError_t e, const char* what) {
  char buf[512];
  snprintf(buf, sizeof buf, "%s: %s", what, hipGetErrorString(e));
  g_last_error = buf;
  g_counters[CNT_HIP_FAIL].fetch_add(1);
  return QA_ERR_HIP;
}

// Debug mode: -1 until first read from QA_DEBUG, then 0 or 1.
std::atomic<int> g_debug{-1};

bool debug_on() {
  int d = g_debug.load(std::memory_order_relaxed);
  if (d < 0) {
    const char* env = std::getenv("QA_DEBUG");
    int want = (env && env[0] && std::strcmp(env, "0") != 0) ? 1 : 0;
    g_debug.compare_exchange_strong(d, want);  // a concurrent qa_set_debug wins
    d = g_debug.load(std::memory_order_relaxed);
  }
  return d == 1;
}

// After a call's launches, in debug mode: wait for them and fail on a pending
// HIP error or a set device error bit (err_word may be NULL).  A stream that
// is being captured is not synchronised.
qa_status debug_check(void* stream, const void* err_word, const char* what) {
  if (!debug_on()) return QA_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  hipError_t e = hipStreamIsCapturing(s, &cap);
  if (e != hipSuccess) return hip_fail(e, "hipStreamIsCapturing");
  if (cap != hipStreamCaptureStatusNone) return QA_OK;
  e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, what);
  e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, what);
  if (err_word) {
    int32_t v = 0;
    e = hipMemcpy(&v, err_word, sizeof v, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(e, "read error word");
    if (v != 0) return fail(QA_ERR_DEVICE, "%s: device error bits 0x%x (debug mode)", what, v);
  }
  return QA_OK;
}

bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool al4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

#define QA_REQUIRE(cond, status, ...) \
  do {                                 \
    if (!(cond)) return fail(status, __VA_ARGS__); \
  } while (0)

qa_status check_cache(const qa_cache* c) {
  QA_REQUIRE(c, QA_ERR_NULL, "cache descriptor is NULL");
  QA_REQUIRE(c->k && c->v, QA_ERR_NULL, "cache k/v memory is NULL");
  QA_REQUIRE(c->head_dim == qa::kHeadDim, QA_ERR_UNSUPPORTED,
             "head_dim %d unsupported (only 128)", c->head_dim);
  QA_REQUIRE(c->batch >= 1 && c->n_kv_heads >= 1 && c->capacity >= 1,
             QA_ERR_SHAPE, "cache batch/n_kv_heads/capacity must be >= 1");
  QA_REQUIRE(al16(c->k) && al16(c->v), QA_ERR_ALIGN,
             "cache k/v must be 16-byte aligned");
  QA_REQUIRE(c->stride_pos >= qa::kHeadDim && c->stride_h >= 1 && c->stride_b >= 1,
             QA_ERR_SHAPE, "cache strides too small");
  QA_REQUIRE(c->stride_pos % 8 == 0 && c->stride_h % 8 == 0 && c->stride_b % 8 == 0,
             QA_ERR_ALIGN, "cache strides must be multiples of 8 elements");
  // a 64-key tile is addressed with 32-bit byte offsets from its first row
  QA_REQUIRE(c->stride_pos <= qa::kMaxStridePos, QA_ERR_SHAPE,
             "cache stride_pos %lld exceeds %lld elements", (long long)c->stride_pos,
             (long long)qa::kMaxStridePos);
  return QA_OK;
}

qa_status check_params(const qa_params* p, const qa_cache* c, int* group) {
  QA_REQUIRE(p, QA_ERR_NULL, "params is NULL");
  QA_REQUIRE(p->n_q_heads >= 1, QA_ERR_SHAPE, "n_q_heads must be >= 1");
  QA_REQUIRE(p->n_q_heads % c->n_kv_heads == 0, QA_ERR_SHAPE,
             "n_q_heads %d is not a multiple of n_kv_heads %d", p->n_q_heads,
             c->n_kv_heads);
  const int G = p->n_q_heads / c->n_kv_heads;
  QA_REQUIRE(G == 1 || G == 2 || G == 4 || G == 8, QA_ERR_UNSUPPORTED,
             "GQA group %d unsupported (1, 2, 4 or 8)", G);
  QA_REQUIRE(std::isfinite(p->rope_theta) && p->rope_theta > 0.0, QA_ERR_SHAPE,
             "rope_theta must be finite and > 0");
  QA_REQUIRE(std::isfinite(p->rms_eps) && p->rms_eps >= 0.0, QA_ERR_SHAPE,
             "rms_eps must be finite and >= 0");
  QA_REQUIRE(std::isfinite(p->softmax_scale) && p->softmax_scale > 0.f,
             QA_ERR_SHAPE, "softmax_scale must be finite and > 0");
  QA_REQUIRE(al16(p->q_norm_w) && al16(p->k_norm_w), QA_ERR_ALIGN,
             "norm weights must be 16-byte aligned");
  *group = G;
  return QA_OK;
}

qa::RopeFreq make_freq(double theta) {
  qa::RopeFreq f;
  for (int i = 0; i < qa::kHalf; ++i)
    f.inv_freq[i] = std::pow(theta, -(2.0 * i) / qa::kHeadDim);
  return f;
}

qa::CacheArgs cache_args(const qa_cache* c) {
  qa::CacheArgs a;
  a.k = static_cast<uint16_t*>(c->k);
  a.v = static_cast<uint16_t*>(c->v);
  a.sb = c->stride_b;
  a.sh = c->stride_h;
  a.sp = c->stride_pos;
  a.capacity = c->capacity;
  return a;
}

int group_of(int n_q_heads, int n_kv_heads) {
  if (n_q_heads < 1 || n_kv_heads < 1 || n_q_heads % n_kv_heads) return 0;
  const int G = n_q_heads / n_kv_heads;
  return (G == 1 || G == 2 || G == 4 || G == 8) ? G : 0;
}

}  // namespace

extern "C" {

qa_status qa_cache_alloc(qa_cache* out, int batch, int n_kv_heads, int capacity,
                         int head_dim, void* k_mem, void* v_mem) {
  QA_REQUIRE(out, QA_ERR_NULL, "out is NULL");
  QA_REQUIRE((k_mem == nullptr) == (v_mem == nullptr), QA_ERR_NULL,
             "pass both k_mem and v_mem, or neither");
  QA_REQUIRE(head_dim == qa::kHeadDim, QA_ERR_UNSUPPORTED,
             "head_dim %d unsupported (only 128)", head_dim);
  QA_REQUIRE(batch >= 1 && n_kv_heads >= 1 && capacity >= 1, QA_ERR_SHAPE,
             "batch, n_kv_heads and capacity must be >= 1");
  QA_REQUIRE(!k_mem || (al16(k_mem) && al16(v_mem)), QA_ERR_ALIGN,
             "k_mem/v_mem must be 16-byte aligned");
  qa_cache c;
  std::memset(&c, 0, sizeof c);
  c.batch = batch;
  c.n_kv_heads = n_kv_heads;
  c.capacity = capacity;
  c.head_dim = head_dim;
  c.stride_pos = head_dim;
  c.stride_h = (int64_t)capacity * head_dim;
  c.stride_b = (int64_t)n_kv_heads * c.stride_h;
  if (k_mem) {
    c.k = k_mem;
    c.v = v_mem;
    c.owns = 0;
  } else {
    const size_t bytes = (size_t)batch * c.stride_b * sizeof(uint16_t);
    hipError_t e = hipMalloc(&c.k, bytes);
    if (e != hipSuccess) return hip_fail(e, "hipMalloc(cache k)");
    e = hipMalloc(&c.v, bytes);
    if (e != hipSuccess) {
      (void)hipFree(c.k);
      return hip_fail(e, "hipMalloc(cache v)");
    }
    c.owns = 1;
  }
  *out = c;
  return QA_OK;
}

qa_status qa_cache_free(qa_cache* c) {
  QA_REQUIRE(c, QA_ERR_NULL, "cache descriptor is NULL");
  if (c->owns) {
    hipError_t e1 = hipFree(c->k), e2 = hipFree(c->v);
    std::memset(c, 0, sizeof *c);
    if (e1 != hipSuccess) return hip_fail(e1, "hipFree(cache k)");
    if (e2 != hipSuccess) return hip_fail(e2, "hipFree(cache v)");
    return QA_OK;
  }
  std::memset(c, 0, sizeof *c);
  return QA_OK;
}

size_t qa_workspace_bytes(int op, int batch, int n_q_heads, int n_kv_heads,
                          int max_ctx, int block_len) {
  const int G = group_of(n_q_heads, n_kv_heads);
  if (!G || batch < 1 || max_ctx < 0) return 0;
  switch (op) {
    case QA_OP_PREFILL:
      return qa::prefill_ws_bytes(max_ctx);
    case QA_OP_DECODE:
      if (max_ctx < 1) return 0;
      return qa::decode_split_layout(batch, n_kv_heads, G, max_ctx).total;
    case QA_OP_VERIFY:
      if (max_ctx < 1 || block_len < 1 || block_len * G > 128) return 0;
      return qa::verify_split_layout(batch, n_kv_heads, G, max_ctx, block_len).total;
    default:
      return 0;
  }
}

qa_status qa_workspace_init(void* ws, size_t ws_bytes, void* stream) {
  QA_REQUIRE(ws, QA_ERR_NULL, "workspace is NULL");
  QA_REQUIRE(al16(ws), QA_ERR_ALIGN, "workspace must be 16-byte aligned");
  QA_REQUIRE(ws_bytes >= qa::kWsHeader && ws_bytes % 16 == 0, QA_ERR_WORKSPACE,
             "workspace must be >= 256 bytes and a multiple of 16");
  hipError_t e = qa::launch_fill_zero(ws, ws_bytes, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "workspace fill kernel");
  g_counters[CNT_WS_INIT].fetch_add(1);
  g_counters[CNT_KERNELS].fetch_add(1);
  return QA_OK;
}

qa_status qa_prefill(const qa_cache* c, const qa_params* p, const void* q,
                     const void* k, const void* v, int64_t q_tok_stride,
                     int64_t kv_tok_stride, const int32_t* cu_seqlens,
                     const int32_t* positions, int n_seq, int total_tokens,
                     int max_seqlen, void* out, float* lse, void* ws,
                     size_t ws_bytes, void* stream) {
  qa_status st = check_cache(c);
  if (st != QA_OK) return st;
  int G = 0;
  st = check_params(p, c, &G);
  if (st != QA_OK) return st;
  QA_REQUIRE(total_tokens >= 0, QA_ERR_SHAPE, "total_tokens must be >= 0");
  if (total_tokens == 0) {
    g_last_error.clear();
    return QA_OK;
  }
  QA_REQUIRE(q && k && v && out && cu_seqlens && positions && ws, QA_ERR_NULL,
             "q, k, v, out, cu_seqlens, positions and ws must be non-NULL");
  QA_REQUIRE(n_seq >= 1 && n_seq <= c->batch, QA_ERR_SHAPE,
             "n_seq %d must be in [1, cache batch %d]", n_seq, c->batch);
  QA_REQUIRE(max_seqlen >= 1, QA_ERR_SHAPE, "max_seqlen must be >= 1");
  QA_REQUIRE(max_seqlen <= c->capacity, QA_ERR_CAPACITY,
             "max_seqlen %d exceeds cache capacity %d", max_seqlen, c->capacity);
  QA_REQUIRE(q_tok_stride >= (int64_t)p->n_q_heads * qa::kHeadDim &&
                 kv_tok_stride >= (int64_t)c->n_kv_heads * qa::kHeadDim,
             QA_ERR_SHAPE, "token strides smaller than one token's heads");
  QA_REQUIRE(q_tok_stride % 8 == 0 && kv_tok_stride % 8 == 0, QA_ERR_ALIGN,
             "token strides must be multiples of 8 elements");
  QA_REQUIRE(al16(q) && al16(k) && al16(v) && al16(out) && al16(ws) && al4(lse) &&
                 al4(cu_seqlens) && al4(positions),
             QA_ERR_ALIGN, "q/k/v/out/ws must be 16-byte aligned");
  QA_REQUIRE(ws_bytes >= qa::prefill_ws_bytes(total_tokens), QA_ERR_WORKSPACE,
             "workspace %zu bytes < %zu needed", ws_bytes,
             qa::prefill_ws_bytes(total_tokens));
  QA_REQUIRE((long long)n_seq * c->n_kv_heads * ((max_seqlen + 127) / 128) * 8 < (1LL << 31),
             QA_ERR_SHAPE, "launch grid too large");

  qa::PrefillArgs a;
  a.c = cache_args(c);
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.q_tok_stride = q_tok_stride;
  a.kv_tok_stride = kv_tok_stride;
  a.cu_seqlens = cu_seqlens;
  a.positions = positions;
  a.n_seq = n_seq;
  a.total_tokens = total_tokens;
  a.max_seqlen = max_seqlen;
  a.n_qtiles = 0;
  a.n_q_heads = p->n_q_heads;
  a.n_kv_heads = c->n_kv_heads;
  a.q_norm_w = static_cast<const uint16_t*>(p->q_norm_w);
  a.k_norm_w = static_cast<const uint16_t*>(p->k_norm_w);
  a.eps = p->rms_eps;
  a.qscale = (float)((double)p->softmax_scale * 1.4426950408889634);
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  a.err = static_cast<int*>(ws);
  a.tile_ctr = static_cast<int*>(ws) + 1;
  a.cs = reinterpret_cast<float2*>(static_cast<char*>(ws) + qa::kWsHeader);
  int nk = 0;
  hipError_t e = qa::launch_prefill(a, make_freq(p->rope_theta), G,
                                    static_cast<hipStream_t>(stream), &nk);
  g_counters[CNT_KERNELS].fetch_add(nk);
  if (e != hipSuccess) return hip_fail(e, "prefill launch");
  g_counters[CNT_PREFILL].fetch_add(1);
  if (qa_status d = debug_check(stream, ws, "prefill"); d != QA_OK) return d;
  g_last_error.clear();
  return QA_OK;
}

static qa_status fill_split_args(qa::DecodeArgs& a, const qa_cache* c,
                                 const qa_params* p, const void* q,
                                 const void* k, const void* v,
                                 const int32_t* pos, int batch, int block_len,
                                 int max_ctx, void* out, float* lse, void* ws,
                                 size_t ws_bytes, const qa::SplitLayout& L) {
  a.c = cache_args(c);
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.positions = pos;
  a.batch = batch;
  a.block_len = block_len;
  a.max_ctx = max_ctx;
  a.n_q_heads = p->n_q_heads;
  a.n_kv_heads = c->n_kv_heads;
  a.keys_per_split = L.keys_per_split;
  a.n_split = L.n_split;
  a.q_norm_w = static_cast<const uint16_t*>(p->q_norm_w);
  a.k_norm_w = static_cast<const uint16_t*>(p->k_norm_w);
  a.eps = p->rms_eps;
  a.qscale = (float)((double)p->softmax_scale * 1.4426950408889634);
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  char* base = static_cast<char*>(ws);
  a.err = reinterpret_cast<int*>(base);
  a.part_m = reinterpret_cast<float*>(base + L.m_off);
  a.part_l = reinterpret_cast<float*>(base + L.l_off);
  a.part_o = reinterpret_cast<float*>(base + L.o_off);
  a.sync = L.sync_off && qa::decode_merges_inline(batch, c->n_kv_heads, L.n_split)
               ? reinterpret_cast<unsigned*>(base + qa::decode_sync_end(ws_bytes))
               : nullptr;
  return QA_OK;
}

qa_status qa_decode(const qa_cache* c, const qa_params* p, const void* q,
                    const void* k, const void* v, const int32_t* positions,
                    int batch, int max_ctx, void* out, float* lse, void* ws,
                    size_t ws_bytes, void* stream) {
  qa_status st = check_cache(c);
  if (st != QA_OK) return st;
  int G = 0;
  st = check_params(p, c, &G);
  if (st != QA_OK) return st;
  QA_REQUIRE(q && k && v && out && positions && ws, QA_ERR_NULL,
             "q, k, v, out, positions and ws must be non-NULL");
  QA_REQUIRE(batch >= 1 && batch <= c->batch, QA_ERR_SHAPE,
             "batch %d must be in [1, cache batch %d]", batch, c->batch);
  QA_REQUIRE(max_ctx >= 1, QA_ERR_SHAPE, "max_ctx must be >= 1");
  QA_REQUIRE(max_ctx <= c->capacity, QA_ERR_CAPACITY,
             "max_ctx %d exceeds cache capacity %d", max_ctx, c->capacity);
  QA_REQUIRE(al16(q) && al16(k) && al16(v) && al16(out) && al16(ws) && al4(lse) &&
                 al4(positions),
             QA_ERR_ALIGN, "q/k/v/out/ws must be 16-byte aligned");
  const qa::SplitLayout L = qa::decode_split_layout(batch, c->n_kv_heads, G, max_ctx);
  QA_REQUIRE(ws_bytes >= L.total, QA_ERR_WORKSPACE,
             "workspace %zu bytes < %zu needed", ws_bytes, L.total);
  qa::DecodeArgs a;
  fill_split_args(a, c, p, q, k, v, positions, batch, 1, max_ctx, out, lse, ws, ws_bytes, L);
  int nk = 0;
  hipError_t e = qa::launch_decode(a, make_freq(p->rope_theta), G,
                                   static_cast<hipStream_t>(stream), &nk);
  g_counters[CNT_KERNELS].fetch_add(nk);
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  g_counters[CNT_DECODE].fetch_add(1);
  if (qa_status d = debug_check(stream, ws, "decode"); d != QA_OK) return d;
  g_last_error.clear();
  return QA_OK;
}

qa_status qa_decode_noalloc(const qa_cache* c, const qa_params* p, const void* q,
                            const void* k, const void* v, const int32_t* positions,
                            int batch, int max_ctx, void* out, float* lse,
                            int32_t* dev_err, void* stream) {
  qa_status st = check_cache(c);
  if (st != QA_OK) return st;
  int G = 0;
  st = check_params(p, c, &G);
  if (st != QA_OK) return st;
  QA_REQUIRE(q && k && v && out && positions, QA_ERR_NULL,
             "q, k, v, out and positions must be non-NULL");
  QA_REQUIRE(batch >= 1 && batch <= c->batch, QA_ERR_SHAPE,
             "batch %d must be in [1, cache batch %d]", batch, c->batch);
  QA_REQUIRE(max_ctx >= 1, QA_ERR_SHAPE, "max_ctx must be >= 1");
  QA_REQUIRE(max_ctx <= c->capacity, QA_ERR_CAPACITY,
             "max_ctx %d exceeds cache capacity %d", max_ctx, c->capacity);
  QA_REQUIRE(al16(q) && al16(k) && al16(v) && al16(out) && al4(lse) && al4(positions) &&
                 al4(dev_err),
             QA_ERR_ALIGN, "q/k/v/out must be 16-byte aligned");
  const qa::SplitLayout L = qa::decode_split_layout(batch, c->n_kv_heads, G, max_ctx);
  const size_t cap_bytes = qa::noalloc_scratch_bytes();
  QA_REQUIRE(L.total <= cap_bytes, QA_ERR_WORKSPACE,
             "decode scratch of %zu bytes exceeds the library's %zu-byte array "
             "(use qa_decode with a workspace)", L.total, cap_bytes);
  hipStream_t s = static_cast<hipStream_t>(stream);
  void* scratch = nullptr;
  hipError_t e = qa::noalloc_scratch(&scratch, s);
  if (e != hipSuccess) return hip_fail(e, "decode scratch");
  qa::DecodeArgs a;
  fill_split_args(a, c, p, q, k, v, positions, batch, 1, max_ctx, out, lse, scratch,
                  cap_bytes, L);
  if (dev_err) a.err = dev_err;
  int nk = 0;
  e = qa::launch_decode(a, make_freq(p->rope_theta), G, s, &nk);
  g_counters[CNT_KERNELS].fetch_add(nk);
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  g_counters[CNT_DECODE].fetch_add(1);
  if (qa_status d = debug_check(stream, dev_err, "decode_noalloc"); d != QA_OK) return d;
  g_last_error.clear();
  return QA_OK;
}

qa_status qa_verify(const qa_cache* c, const qa_params* p, const void* q,
                    const void* k, const void* v, const int32_t* start_pos,
                    int batch, int block_len, int max_ctx, void* out,
                    float* lse, void* ws, size_t ws_bytes, void* stream) {
  qa_status st = check_cache(c);
  if (st != QA_OK) return st;
  int G = 0;
  st = check_params(p, c, &G);
  if (st != QA_OK) return st;
  QA_REQUIRE(q && k && v && out && start_pos && ws, QA_ERR_NULL,
             "q, k, v, out, start_pos and ws must be non-NULL");
  QA_REQUIRE(batch >= 1 && batch <= c->batch, QA_ERR_SHAPE,
             "batch %d must be in [1, cache batch %d]", batch, c->batch);
  QA_REQUIRE(block_len >= 1 && block_len * G <= 128, QA_ERR_SHAPE,
             "block_len %d: need 1 <= block_len and block_len*G <= 128", block_len);
  QA_REQUIRE(max_ctx >= block_len, QA_ERR_SHAPE, "max_ctx must be >= block_len");
  QA_REQUIRE(max_ctx <= c->capacity, QA_ERR_CAPACITY,
             "max_ctx %d exceeds cache capacity %d", max_ctx, c->capacity);
  QA_REQUIRE(al16(q) && al16(k) && al16(v) && al16(out) && al16(ws) && al4(lse) &&
                 al4(start_pos),
             QA_ERR_ALIGN, "q/k/v/out/ws must be 16-byte aligned");
  const qa::SplitLayout L =
      qa::verify_split_layout(batch, c->n_kv_heads, G, max_ctx, block_len);
  QA_REQUIRE(ws_bytes >= L.total, QA_ERR_WORKSPACE,
             "workspace %zu bytes < %zu needed", ws_bytes, L.total);
  qa::DecodeArgs a;
  fill_split_args(a, c, p, q, k, v, start_pos, batch, block_len, max_ctx, out, lse,
                  ws, ws_bytes, L);
  int nk = 0;
  hipError_t e = qa::launch_verify(a, make_freq(p->rope_theta), G,
                                   static_cast<hipStream_t>(stream), &nk);
  g_counters[CNT_KERNELS].fetch_add(nk);
  if (e != hipSuccess) return hip_fail(e, "verify launch");
  g_counters[CNT_VERIFY].fetch_add(1);
  if (qa_status d = debug_check(stream, ws, "verify"); d != QA_OK) return d;
  g_last_error.clear();
  return QA_OK;
}

qa_status qa_rmsnorm_hidden(const void* x, void* residual, const void* weight,
                            int n_tokens, int hidden, double eps, void* out,
                            void* stream) {
  QA_REQUIRE((x && out) || n_tokens == 0, QA_ERR_NULL, "x and out must be non-NULL");
  QA_REQUIRE(n_tokens >= 0, QA_ERR_SHAPE, "n_tokens %d < 0", n_tokens);
  QA_REQUIRE(hidden >= 8 && hidden % 8 == 0, QA_ERR_SHAPE,
             "hidden %d must be a positive multiple of 8", hidden);
  QA_REQUIRE(hidden <= 64 * 8 * qa::kNormMaxChunks, QA_ERR_UNSUPPORTED,
             "hidden %d exceeds %d", hidden, 64 * 8 * qa::kNormMaxChunks);
  QA_REQUIRE(eps >= 0.0 && eps < 1.0e30, QA_ERR_SHAPE, "eps must be finite and >= 0");
  QA_REQUIRE(al16(x) && al16(out) && al16(residual) && al16(weight), QA_ERR_ALIGN,
             "x/residual/weight/out must be 16-byte aligned");
  qa::NormArgs a;
  a.x = static_cast<const uint16_t*>(x);
  a.res = static_cast<uint16_t*>(residual);
  a.w = static_cast<const uint16_t*>(weight);
  a.out = static_cast<uint16_t*>(out);
  a.n_tokens = n_tokens;
  a.hidden = hidden;
  a.eps = eps;
  hipError_t e = qa::launch_rmsnorm_hidden(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "rmsnorm launch");
  if (n_tokens > 0) g_counters[CNT_KERNELS].fetch_add(1);
  if (qa_status d = debug_check(stream, nullptr, "rmsnorm_hidden"); d != QA_OK) return d;
  g_last_error.clear();
  return QA_OK;
}

qa_status qa_attn_epilogue(const void* o, int64_t o_tok_stride, const void* w_o,
                           void* residual, const void* norm_w, int n_tokens, int in_dim,
                           int hidden, double eps, void* out, void* stream) {
  QA_REQUIRE(n_tokens >= 0, QA_ERR_SHAPE, "n_tokens %d < 0", n_tokens);
  if (n_tokens == 0) {
    g_last_error.clear();
    return QA_OK;
  }
  QA_REQUIRE(o && w_o && residual && out, QA_ERR_NULL,
             "o, w_o, residual and out must be non-NULL");
  QA_REQUIRE(in_dim >= qa::kEpBK && in_dim % qa::kEpBK == 0, QA_ERR_UNSUPPORTED,
             "in_dim %d must be a positive multiple of %d", in_dim, qa::kEpBK);
  QA_REQUIRE(hidden >= qa::kEpBN && hidden % qa::kEpBN == 0, QA_ERR_UNSUPPORTED,
             "hidden %d must be a positive multiple of %d", hidden, qa::kEpBN);
  QA_REQUIRE(hidden <= 64 * 8 * qa::kNormMaxChunks, QA_ERR_UNSUPPORTED,
             "hidden %d exceeds %d", hidden, 64 * 8 * qa::kNormMaxChunks);
  QA_REQUIRE(o_tok_stride >= in_dim && o_tok_stride % 8 == 0, QA_ERR_SHAPE,
             "o_tok_stride %lld must be >= in_dim and a multiple of 8",
             (long long)o_tok_stride);
  QA_REQUIRE(eps >= 0.0 && eps < 1.0e30, QA_ERR_SHAPE, "eps must be finite and >= 0");
  QA_REQUIRE(al16(o) && al16(w_o) && al16(residual) && al16(norm_w) && al16(out),
             QA_ERR_ALIGN, "o/w_o/residual/norm_w/out must be 16-byte aligned");
  QA_REQUIRE(out != residual, QA_ERR_SHAPE, "out may not alias residual");
  qa::EpilogueArgs a;
  a.o = static_cast<const uint16_t*>(o);
  a.o_stride = o_tok_stride;
  a.w = static_cast<const uint16_t*>(w_o);
  a.res = static_cast<uint16_t*>(residual);
  a.n_tokens = n_tokens;
  a.in_dim = in_dim;
  a.hidden = hidden;
  qa::NormArgs n;
  n.x = static_cast<const uint16_t*>(residual);
  n.res = nullptr;
  n.w = static_cast<const uint16_t*>(norm_w);
  n.out = static_cast<uint16_t*>(out);
  n.n_tokens = n_tokens;
  n.hidden = hidden;
  n.eps = eps;
  int nk = 0;
  hipError_t e = qa::launch_attn_epilogue(a, n, static_cast<hipStream_t>(stream), &nk);
  g_counters[CNT_KERNELS].fetch_add(nk);
  if (e != hipSuccess) return hip_fail(e, "epilogue launch");
  if (qa_status d = debug_check(stream, nullptr, "attn_epilogue"); d != QA_OK) return d;
  g_last_error.clear();
  return QA_OK;
}

qa_status qa_copy(const void* src, void* dst, size_t bytes, void* stream) {
  QA_REQUIRE(src && dst, QA_ERR_NULL, "src/dst NULL");
  QA_REQUIRE(al16(src) && al16(dst) && bytes % 16 == 0, QA_ERR_ALIGN,
             "copy needs 16-byte aligned pointers and size");
  hipError_t e = qa::launch_copy(src, dst, bytes, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "copy launch");
  g_counters[CNT_COPY].fetch_add(1);
  g_counters[CNT_KERNELS].fetch_add(1);
  return debug_check(stream, nullptr, "copy");
}

const char* qa_status_str(qa_status s) {
  switch (s) {
    case QA_OK: return "QA_OK";
    case QA_ERR_NULL: return "QA_ERR_NULL";
    case QA_ERR_SHAPE: return "QA_ERR_SHAPE";
    case QA_ERR_UNSUPPORTED: return "QA_ERR_UNSUPPORTED";
    case QA_ERR_ALIGN: return "QA_ERR_ALIGN";
    case QA_ERR_CAPACITY: return "QA_ERR_CAPACITY";
    case QA_ERR_WORKSPACE: return "QA_ERR_WORKSPACE";
    case QA_ERR_HIP: return "QA_ERR_HIP";
    case QA_ERR_DEVICE: return "QA_ERR_DEVICE";
  }
  return "QA_ERR_UNKNOWN";
}

const char* qa_last_error(void) { return g_last_error.c_str(); }

void qa_set_debug(int on) { g_debug.store(on ? 1 : 0); }

void qa_get_counters(uint64_t out[8]) {
  for (int i = 0; i < 8; ++i) out[i] = g_counters[i].load();
}

void qa_reset_counters(void) {
  for (int i = 0; i < 8; ++i) g_counters[i].store(0);
}

qa_status qa_device_error(void* ws, void* stream, int32_t* code) {
  QA_REQUIRE(ws && code, QA_ERR_NULL, "ws/code NULL");
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
  int32_t v = 0;
  e = hipMemcpy(&v, ws, sizeof v, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "read error word");
  const int32_t zero = 0;
  e = hipMemcpy(ws, &zero, sizeof zero, hipMemcpyHostToDevice);
  if (e != hipSuccess) return hip_fail(e, "clear error word");
  *code = v;
  return QA_OK;
}

}  // extern "C"
