// Internal declarations shared by the host library and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "merge_count.h"

namespace qa {

constexpr int kHeadDim = 128;
constexpr int kHalf = 64;        // rotation pairs per head
constexpr int kKeyTile = 64;     // keys per LDS tile in the MFMA kernels
constexpr size_t kWsHeader = 256;  // error word + reserved

// Rotation frequencies theta^(-2i/128), computed on the host in fp64 and
// passed by value (kernel arguments), so every kernel uses the same values.
struct RopeFreq {
  double inv_freq[kHalf];
};

// ---- workspace layout --------------------------------------------------------
//   [0, 256)                 int32 error word at 0; prefill: int32 q-tile
//                            counter at 4 (zeroed by every prefill call)
//   prefill: + cos/sin table float2 [total_tokens][64]
//   decode / verify: + fp32 m, l [batch][n_kv][n_split][rows] each
//                    + fp32 o   [batch][n_kv][n_split][rows][128]
// rows = G (decode) or block_len*G (verify).
inline size_t round256(size_t x) { return (x + 255) & ~size_t(255); }

struct SplitLayout {
  int keys_per_split;
  int n_split;
  size_t m_off, l_off, o_off, total;
  size_t sync_off = 0;  // decode only: the in-launch merge counters
};

// Decode: keys per split-K workgroup, a multiple of 16 (one score tile) of
// at most kDecodeMaxTiles tiles.  A workgroup is kDecodeWaves waves, one
// workgroup per CU (two or three waves per SIMD).  Nine rather than eight: a
// split of the 4 x 8-pair batch at 2049-2176 slots runs 16-17 tiles, which
// on eight waves leaves one wave a third tile, loaded only after its first is
// used; on nine no wave has more than two, both loaded at entry (11.87 ->
// 11.67 us per call).  The split count aims at
// kDecodeBlocks workgroups in all, so every CU streams the same number of
// cache bytes in one round: a grid a few workgroups over a multiple of the
// CU count leaves those CUs another workgroup to stream after the rest have
// finished.  Fewer, larger workgroups also halve the partials the merge reads
// against four-wave workgroups at two per CU.  The split is a function of the
// launch sizes only (never of device-side positions), so graphs stay valid.
constexpr int kDecodeWaves = 9;
constexpr int kDecodeBlocks = 256;
constexpr int kDecodeMaxTiles = 4 * kDecodeWaves;  // at most 4 tiles per wave
inline int decode_keys_per_split(int batch, int n_kv, int max_ctx) {
  long pairs = (long)batch * n_kv;
  long want = kDecodeBlocks / pairs;  // splits per (sequence, kv head)
  if (want < 1) want = 1;
  long ks = (max_ctx + want - 1) / want;
  ks = (ks + 15) / 16 * 16;
  if (ks < 16) ks = 16;
  if (ks > 16 * kDecodeMaxTiles) ks = 16 * kDecodeMaxTiles;
  return (int)ks;
}

// extra: partials beyond the cache splits (decode adds one for the new token).
inline SplitLayout split_layout(int batch, int n_kv, int rows, int max_ctx,
                                int keys_per_split, int extra = 0) {
  SplitLayout L;
  L.keys_per_split = keys_per_split;
  L.n_split = (max_ctx + keys_per_split - 1) / keys_per_split;
  if (L.n_split < 1) L.n_split = 1;
  L.n_split += extra;
  size_t pairs = (size_t)batch * n_kv;
  size_t nrow = pairs * L.n_split * rows;
  L.m_off = kWsHeader;
  L.l_off = L.m_off + round256(nrow * sizeof(float));
  L.o_off = L.l_off + round256(nrow * sizeof(float));
  L.total = L.o_off + round256(nrow * kHeadDim * sizeof(float));
  return L;
}

// Decode partials: one per cache split (the rows before the new slot; split
// 0 also takes the new token's key).  Then room for one 128-byte line per (sequence, kv head)
// holding the arrival counter of the in-launch merge.  The counters are
// placed from the END of the caller's workspace downwards (pair p at
// end - 128 (p + 1), end = ws_bytes rounded down to 128), so a workspace
// reused for a smaller batch or context finds the same, zeroed, counters.
// They are zero after qa_workspace_init and returned to zero by every call.
constexpr size_t kSyncLine = 128;
constexpr int kSyncWords = (int)(kSyncLine / 4);
inline SplitLayout decode_split_layout(int batch, int n_kv, int G, int max_ctx) {
  const int rows_before = max_ctx > 1 ? max_ctx - 1 : 1;
  SplitLayout L = split_layout(batch, n_kv, G, rows_before,
                               decode_keys_per_split(batch, n_kv, rows_before));
  L.sync_off = L.total;
  L.total = L.sync_off + round256((size_t)batch * n_kv * kSyncLine);
  return L;
}
// End of the counter block for a workspace of ws_bytes (bytes from its start).
inline size_t decode_sync_end(size_t ws_bytes) { return ws_bytes & ~(kSyncLine - 1); }

// The in-launch merge needs the pairs to fill whole rounds of the 8-XCD deal
// and at most 127 splits (the counter's fields); other launches merge in a
// second kernel.
inline bool decode_merges_inline(int batch, int n_kv, int n_split) {
  return ((long)batch * n_kv) % 8 == 0 && n_split <= kInlineMaxSplits;
}

// Prefill: the header, then the cos/sin table float2 [total_tokens][64] that
// the K/V prologue writes for the queries.
inline size_t prefill_ws_bytes(int total_tokens) {
  return kWsHeader + round256((size_t)total_tokens * kHalf * sizeof(float2));
}

// ---- kernel argument blocks ----------------------------------------------------
// Largest cache stride_pos (elements): 64 rows of a key tile must span less
// than 2^31 bytes so the tile loader's per-lane offsets fit 32 bits.
constexpr int64_t kMaxStridePos = int64_t(1) << 23;

struct CacheArgs {
  uint16_t* k;
  uint16_t* v;
  int64_t sb, sh, sp;  // element strides
  int capacity;
};

struct PrefillArgs {
  CacheArgs c;
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  int64_t q_tok_stride, kv_tok_stride;
  const int32_t* cu_seqlens;
  const int32_t* positions;
  int n_seq, total_tokens, max_seqlen, n_qtiles;
  int n_q_heads, n_kv_heads;
  const uint16_t* q_norm_w;
  const uint16_t* k_norm_w;
  double eps;
  float qscale;  // softmax_scale * log2(e), folded into q'
  uint16_t* out;
  float* lse;
  int* err;
  int* tile_ctr;  // per-XCD q-tile counters of the attention grid (workspace header)
  float2* cs;  // cos/sin table in the workspace, [total_tokens][64]
};

struct DecodeArgs {
  CacheArgs c;
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* positions;  // decode: position per sequence; verify: start
  int batch, block_len, max_ctx;
  int n_q_heads, n_kv_heads;
  int keys_per_split, n_split;
  const uint16_t* q_norm_w;
  const uint16_t* k_norm_w;
  double eps;
  float qscale;
  uint16_t* out;
  float* lse;
  int* err;
  float* part_m;
  float* part_l;
  float* part_o;
  unsigned* sync;  // decode: END of the merge counters (pair p's at sync - kSyncWords (p+1));
                   // NULL: merge kernel
};

// Attention epilogue GEMM: 256 x 128 output tiles, K in steps of 64.  Up to
// kEpSmallT tokens use the streaming kernel instead: kEpSmallN output features
// per workgroup.
constexpr int kEpBM = 256, kEpBN = 128, kEpBK = 64;
constexpr int kEpSmallT = 32, kEpSmallN = 16;

struct EpilogueArgs {
  const uint16_t* o;  // attention output [n_tokens][in_dim], token stride o_stride
  int64_t o_stride;
  const uint16_t* w;  // output projection weight [hidden][in_dim]
  uint16_t* res;      // residual stream [n_tokens][hidden], updated in place
  int n_tokens, in_dim, hidden;
};

// ---- launchers (return the hipError_t of the launch) ------------------------------
hipError_t launch_prefill(const PrefillArgs& a, const RopeFreq& f, int group,
                          hipStream_t s, int* n_kernels);
hipError_t launch_decode(const DecodeArgs& a, const RopeFreq& f, int group,
                         hipStream_t s, int* n_kernels);
hipError_t launch_verify(const DecodeArgs& a, const RopeFreq& f, int group,
                         hipStream_t s, int* n_kernels);
hipError_t launch_merge(const DecodeArgs& a, int group, hipStream_t s);
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s);
struct NormArgs;
hipError_t launch_attn_epilogue(const EpilogueArgs& a, const NormArgs& n, hipStream_t s,
                                int* n_kernels);
// qa_decode_noalloc's scratch array (noalloc.hip)
size_t noalloc_scratch_bytes();
hipError_t noalloc_scratch(void** out, hipStream_t s);
hipError_t launch_copy(const void* src, void* dst, size_t bytes, hipStream_t s);

}  // namespace qa
