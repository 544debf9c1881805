// Workspace layout of qa_verify (host side).
#pragma once

#include "qa_internal.h"

namespace qa {

// Per (sequence, kv head) n_split - 1 workgroups stream the cache slots
// before the block (near-equal runs of whole 64-key tiles, cut on the device
// from the start position) and one more writes the block's slots and attends
// to them alone, so its prologue is not followed by a long run of cache
// tiles.  About one workgroup per CU in total (the MFMA kernel's registers
// and LDS leave no room for a second); the split count is a function of the
// launch sizes only.
inline int verify_old_splits(int batch, int n_kv, int max_ctx, int block_len) {
  long pairs = (long)batch * n_kv;
  long want = pairs >= 128 ? 1 : 256 / pairs - 1;
  long tiles = ((long)max_ctx - block_len + kKeyTile - 1) / kKeyTile;
  if (want > tiles) want = tiles;
  return want < 1 ? 1 : (int)want;
}

// The old-slot splits' partials, then the block's (keys_per_split is not
// used by verify).
inline SplitLayout verify_split_layout(int batch, int n_kv, int G, int max_ctx,
                                       int block_len) {
  const int n_old = verify_old_splits(batch, n_kv, max_ctx, block_len);
  return split_layout(batch, n_kv, block_len * G, n_old, 1, 1);  // n_old + 1 splits
}

}  // namespace qa
