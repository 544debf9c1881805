// Hidden-state RMSNorm: declarations shared by the host library and
// rmsnorm.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qa {

// Rows of `hidden` bf16 values, hidden a multiple of 8 and at most
// 64 * 8 * kNormMaxChunks (one wave per row, kNormMaxChunks 16-byte pieces
// per lane).
constexpr int kNormMaxChunks = 16;
// Batches up to this many rows run one workgroup per row.
constexpr int kNormRowTokens = 512;

struct NormArgs {
  const uint16_t* x;
  uint16_t* res;        // residual stream in/out, or NULL
  const uint16_t* w;    // weight [hidden] or NULL (ones)
  uint16_t* out;
  int n_tokens, hidden;
  double eps;
};

hipError_t launch_rmsnorm_hidden(const NormArgs& a, hipStream_t s);

}  // namespace qa
