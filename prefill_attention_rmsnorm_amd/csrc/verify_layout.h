// Workspace layout of qa_verify (host side).
#pragma once

#include "qa_internal.h"

namespace qa {

// Per (sequence, kv head) n_split - 1 workgroups stream the cache slots
// before the block (near-equal runs of whole 64-key tiles, cut on the device
// from the start position) and one more writes the block's slots and attends
// to them alone, so its prologue is not followed by a long run of cache
// tiles.  The workgroup count aims at filling every CU once: the MFMA
// kernel's registers allow one wave per SIMD (so 4 / waves workgroups per
// CU), and its LDS (three 16 KB tiles plus a fourth that also holds the
// queries' cos/sin rows, 512 bytes per draft token) allows two workgroups
// per CU when the rows fit in 16 KB (G >= 4), else one.  The split count is
// a function of the launch sizes only.
inline int verify_waves(int rows) { return rows <= 32 ? 1 : rows <= 64 ? 2 : 4; }

// Blocks of up to this many tokens on 2 or 4 waves stream their old slots
// through the four-stage K/V ring (eight 16 KB tiles and the cos/sin rows:
// 144 KB of LDS, one workgroup per CU).  One wave would need 6 x 16 copies in
// flight, more than its memory counter holds.
constexpr int kVerifyRingTokens = 32;
inline bool verify_uses_ring(int G, int block_len) {
  return verify_waves(block_len * G) >= 2 && block_len <= kVerifyRingTokens;
}

inline int verify_workgroups_per_cu(int G, int block_len) {
  const int by_simd = 4 / verify_waves(block_len * G);
  const int by_lds = verify_uses_ring(G, block_len) ? 1 : G >= 4 ? 2 : 1;
  return by_simd < by_lds ? by_simd : by_lds;
}

constexpr int kVerifyCUs = 256;
// Workgroups per CU the split count aims at (at most what fits).
constexpr int kVerifyTargetPerCU = 1;

inline int verify_old_splits(int batch, int n_kv, int G, int max_ctx, int block_len) {
  const long pairs = (long)batch * n_kv;
  const int fit = verify_workgroups_per_cu(G, block_len);
  const long slots =
      (long)kVerifyCUs * (fit < kVerifyTargetPerCU ? fit : kVerifyTargetPerCU);
  long want = pairs * 2 > slots ? 1 : slots / pairs - 1;
  const long tiles = ((long)max_ctx - block_len + kKeyTile - 1) / kKeyTile;
  if (want > tiles) want = tiles;
  return want < 1 ? 1 : (int)want;
}

// The old-slot splits' partials, then the block's (keys_per_split is not
// used by verify).  The partials are merged by merge.hip in a second launch:
// a verify partial is 64 rows of 130 floats per split, so one workgroup
// reading a pair's partials back (as decode's in-launch merge does for its
// 4 rows) would take longer than the second launch.
inline SplitLayout verify_split_layout(int batch, int n_kv, int G, int max_ctx,
                                       int block_len) {
  const int n_old = verify_old_splits(batch, n_kv, G, max_ctx, block_len);
  return split_layout(batch, n_kv, block_len * G, n_old, 1, 1);  // n_old + 1 splits
}

}  // namespace qa
