// Prompt prefill on gfx950: K/V prologue + causal GQA flash attention.
//
// "dryft-flash-infer" agent guide, Where the wins are: prefill is a large share
// of the time at prompts of 512-2048 tokens; RMSNorm and rotary embedding are
// fused; the cache is preallocated and strided.  Kernel 1 writes the cache
// (fp64 K prologue, one RNE to bf16) and a cos/sin table for the queries;
// kernel 2 normalises and rotates q while loading it and runs the MFMA flash
// loop over the cache.
#include <climits>

#include "attn_tile.h"
#include "qa.h"

namespace qa {

// One wave per token: cos/sin of its angles, then k' and v of every KV head.
__global__ __launch_bounds__(256) void kv_prologue_kernel(PrefillArgs a,
                                                          RopeFreq f) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= a.total_tokens) return;
  const int pos = a.positions[t];

  double sn = 0.0, cn = 1.0;
  {
    const double ang = (double)pos * f.inv_freq[lane];
    sincos(ang, &sn, &cn);
  }
  a.cs[(size_t)t * kHalf + lane] = make_float2((float)cn, (float)sn);

  // sequence owning token t: the last i with cu[i] <= t
  int lo = 0, hi = a.n_seq;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (a.cu_seqlens[mid] <= t) lo = mid; else hi = mid;
  }
  const int c0 = a.cu_seqlens[lo], c1 = a.cu_seqlens[lo + 1];
  if (!(c0 <= t && t < c1 && c1 - c0 <= a.max_seqlen)) {
    if (lane == 0) flag_error(a.err, QA_DEVERR_SEQLENS);
    return;
  }
  if (pos < 0 || pos >= a.c.capacity) {
    if (lane == 0) flag_error(a.err, QA_DEVERR_POSITION);
    return;
  }
  const double w_lo = a.k_norm_w ? (double)bf_to_f(a.k_norm_w[lane]) : 1.0;
  const double w_hi = a.k_norm_w ? (double)bf_to_f(a.k_norm_w[lane + 64]) : 1.0;
  const size_t row0 = (size_t)lo * a.c.sb + (size_t)pos * a.c.sp;
  for (int g = 0; g < a.n_kv_heads; ++g) {
    const uint16_t* kr = a.k + (size_t)t * a.kv_tok_stride + (size_t)g * kHeadDim;
    uint16_t o0, o1;
    kprime_pair(kr[lane], kr[lane + 64], w_lo, w_hi, a.eps, cn, sn, &o0, &o1);
    uint16_t* ck = a.c.k + row0 + (size_t)g * a.c.sh;
    ck[lane] = o0;
    ck[lane + 64] = o1;
    const uint32_t* vr = reinterpret_cast<const uint32_t*>(
        a.v + (size_t)t * a.kv_tok_stride + (size_t)g * kHeadDim);
    reinterpret_cast<uint32_t*>(a.c.v + row0 + (size_t)g * a.c.sh)[lane] = vr[lane];
  }
}

// Workgroup = 4 waves = 128 query rows = G heads x (128/G) tokens of one
// sequence and KV head.  Blocks are ordered heaviest q-tile first; when the
// number of (sequence, kv head) pairs is a multiple of 8, all tiles of a pair
// land on one XCD (the hardware deals workgroup ids to the 8 XCDs round
// robin), so its K/V stay in that XCD's L2.
template <int G>
__global__ __launch_bounds__(256, 2) void prefill_attn_kernel(PrefillArgs a) {
  constexpr int TQ = 128 / G;
  __shared__ __attribute__((aligned(16))) unsigned char stage0[kStageBytes];
  __shared__ __attribute__((aligned(16))) unsigned char stage1[kStageBytes];

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int j = l & 31, h2 = l >> 5;

  const int n_pairs = a.n_seq * a.n_kv_heads;
  const int x = blockIdx.x;
  int pair, qt_rev;
  if ((n_pairs & 7) == 0) {
    const int ppx = n_pairs >> 3, slot = x >> 3;
    pair = (slot % ppx) * 8 + (x & 7);
    qt_rev = slot / ppx;
  } else {
    pair = x % n_pairs;
    qt_rev = x / n_pairs;
  }
  const int seq = pair / a.n_kv_heads, g = pair % a.n_kv_heads;
  const int qt = a.n_qtiles - 1 - qt_rev;

  const int s0 = a.cu_seqlens[seq], s1 = a.cu_seqlens[seq + 1];
  if (s0 < 0 || s1 < s0 || s1 > a.total_tokens || s1 - s0 > a.max_seqlen) {
    if (tid == 0) flag_error(a.err, QA_DEVERR_SEQLENS);
    return;
  }
  const int tok0 = s0 + qt * TQ;
  const int n_tok = min(TQ, s1 - tok0);
  if (n_tok <= 0) return;

  // this lane's query column
  const int r = 32 * w + j;
  const int hl = r / TQ, tl = r % TQ;
  const int h = g * G + hl;
  const bool tok_ok = tl < n_tok;
  const int t = tok0 + tl;

  // Positions of the block's tokens: every wave reads all of them (TQ <= 128)
  // and reduces in registers, so no LDS round trip or barrier is needed.
  // The q-side reads go out together with them.
  int pv0 = -1, pv1 = -1;
  if (l < n_tok) pv0 = a.positions[tok0 + l];
  if (TQ > 64 && l + 64 < n_tok) pv1 = a.positions[tok0 + l + 64];
  QPrologue qp;
  qp.load(a.q + (size_t)t * a.q_tok_stride + (size_t)h * kHeadDim, tok_ok,
          a.cs + (size_t)(tok_ok ? t : 0) * kHalf, a.q_norm_w, h2);

  const int cap = a.c.capacity;
  const bool v0 = pv0 >= 0 && pv0 < cap, v1 = pv1 >= 0 && pv1 < cap;
  int kv_end = max(v0 ? pv0 + 1 : 0, v1 ? pv1 + 1 : 0);
  int pmin = min(v0 ? pv0 : INT_MAX, v1 ? pv1 : INT_MAX);
#pragma unroll
  for (int sh = 1; sh < 64; sh <<= 1) {
    kv_end = max(kv_end, __shfl_xor(kv_end, sh));
    pmin = min(pmin, __shfl_xor(pmin, sh));
  }
  // wave-uniform (the tile loader's buffer descriptors must live in SGPRs)
  kv_end = __builtin_amdgcn_readfirstlane(kv_end);
  pmin = __builtin_amdgcn_readfirstlane(pmin);
  const int pa = __shfl(pv0, tl & 63), pb = __shfl(pv1, tl & 63);
  int p = !tok_ok ? -1 : (tl < 64 ? pa : pb);
  const bool q_ok = tok_ok && p >= 0 && p < cap;
  if (!q_ok) p = kv_end - 1;  // sees every key; its output is not kept

  uint16_t* orow = a.out + ((size_t)t * a.n_q_heads + h) * kHeadDim;
  if (kv_end == 0) {  // no valid position in the tile
    if (tok_ok) {
      const u32x2 z = {0u, 0u};
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4)
          *reinterpret_cast<u32x2*>(orow + 32 * db + 8 * a4 + 4 * h2) = z;
      if (a.lse && h2 == 0) a.lse[(size_t)t * a.n_q_heads + h] = 0.f;
    }
    return;
  }

  const uint16_t* kbase = a.c.k + (size_t)seq * a.c.sb + (size_t)g * a.c.sh;
  const uint16_t* vbase = a.c.v + (size_t)seq * a.c.sb + (size_t)g * a.c.sh;

  TileLoader<4> ld;
  ld.init(__builtin_amdgcn_readfirstlane(w), l, a.c.sp);
  load_first(ld, stage0, kbase, vbase, a.c.sp, 0, kv_end);

  u32x4 qb[8];
  qp.compute((float)a.eps, a.qscale, qb);

  WaveAttn st;
  st.init(l);
  // tiles wholly at or below the smallest position need no mask
  const int n_unmasked = (pmin + 1) / kKeyTile;
  attend_tiles(st, ld, stage0, stage1, kbase, vbase, a.c.sp, 0, kv_end, n_unmasked, qb,
               p, h2);

  const float lt = st.lsum + __shfl_xor(st.lsum, 32);
  const float inv = q_ok ? 1.0f / lt : 0.f;
  if (tok_ok) {
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        u32x2 pr = {0u, 0u};
        if (q_ok) {
          pr[0] = pack_bf16x2(st.o[db][4 * a4] * inv, st.o[db][4 * a4 + 1] * inv);
          pr[1] = pack_bf16x2(st.o[db][4 * a4 + 2] * inv, st.o[db][4 * a4 + 3] * inv);
        }
        *reinterpret_cast<u32x2*>(orow + 32 * db + 8 * a4 + 4 * h2) = pr;
      }
    if (a.lse && h2 == 0)
      a.lse[(size_t)t * a.n_q_heads + h] =
          q_ok ? (st.m + __log2f(lt)) * kLn2 : 0.f;
  }
}

hipError_t launch_prefill(const PrefillArgs& a0, const RopeFreq& f, int group,
                          hipStream_t s, int* n_kernels) {
  PrefillArgs a = a0;
  *n_kernels = 0;
  if (a.total_tokens == 0) return hipSuccess;
  hipLaunchKernelGGL(kv_prologue_kernel, dim3((a.total_tokens + 3) / 4),
                     dim3(256), 0, s, a, f);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  ++*n_kernels;
  const int tq = 128 / group;
  a.n_qtiles = (a.max_seqlen + tq - 1) / tq;
  const dim3 grid((unsigned)(a.n_seq * a.n_kv_heads * a.n_qtiles));
  switch (group) {
    case 1: hipLaunchKernelGGL(prefill_attn_kernel<1>, grid, dim3(256), 0, s, a); break;
    case 2: hipLaunchKernelGGL(prefill_attn_kernel<2>, grid, dim3(256), 0, s, a); break;
    case 4: hipLaunchKernelGGL(prefill_attn_kernel<4>, grid, dim3(256), 0, s, a); break;
    case 8: hipLaunchKernelGGL(prefill_attn_kernel<8>, grid, dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  e = hipGetLastError();
  if (e == hipSuccess) ++*n_kernels;
  return e;
}

}  // namespace qa
