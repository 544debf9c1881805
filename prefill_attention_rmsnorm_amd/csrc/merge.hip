// Log-sum-exp merge of split-K partials (verify, and decode launches that do
// not merge inside their own launch).
//
// Each split workgroup of decode.hip / verify.hip wrote, per query row, the
// row's max m (log2 units), sum l and unnormalised output o over its keys.
// For a row, with M = max_s m_s:
//   out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s,
//   lse = (M + log2 sum_s 2^(m_s - M) l_s) * ln 2.
// The merge runs as its own launch, so the kernel boundary (not per-workgroup
// device-scope fences) makes the partials visible.  Splits are combined in
// split order; results do not depend on scheduling.
#include "qa.h"
#include "qa_device.h"

namespace qa {

// grid: (ceil(rows*32 / 128), batch*n_kv_heads); thread = (row, 4 dims)
__global__ __launch_bounds__(128) void merge_kernel(DecodeArgs a, int G) {
  const int rows = a.block_len * G;
  const int item = blockIdx.x * 128 + threadIdx.x;
  if (item >= rows * 32) return;
  const int pair = blockIdx.y;
  const int b = pair / a.n_kv_heads, g = pair % a.n_kv_heads;
  const int rr = item >> 5, d4 = (item & 31) * 4;
  const size_t r0 = (size_t)pair * a.n_split * rows + rr;
  const float* pm = a.part_m + r0;
  const float* pl = a.part_l + r0;
  const float* po = a.part_o + r0 * kHeadDim + d4;
  auto load = [&](int s, float& m, float& l, float4& o) {
    m = pm[(size_t)s * rows];
    l = pl[(size_t)s * rows];
    o = *reinterpret_cast<const float4*>(po + (size_t)s * rows * kHeadDim);
  };
  // loads in flight per batch: the split count rounded up to 4, 8 or 16, so
  // that no batch carries more clamped duplicate loads than it must
  const int ns = a.n_split;
  const MergeOut mo = ns <= 4   ? merge_splits<4>(ns, load)
                      : ns <= 8 ? merge_splits<8>(ns, load)
                                : merge_splits<16>(ns, load);
  const int n = a.block_len;
  const int hl = rr / n, ti = rr % n;
  const size_t orow = (((size_t)b * n + ti) * a.n_q_heads + g * G + hl) * kHeadDim;
  store_merged(mo, false, a.out + orow + d4,
               a.lse && d4 == 0 ? a.lse + ((size_t)b * n + ti) * a.n_q_heads + g * G + hl
                                : nullptr);
}

hipError_t launch_merge(const DecodeArgs& a, int group, hipStream_t s) {
  const int rows = a.block_len * group;
  const dim3 grid((rows * 32 + 127) / 128, a.batch * a.n_kv_heads);
  hipLaunchKernelGGL(merge_kernel, grid, dim3(128), 0, s, a, group);
  return hipGetLastError();
}

}  // namespace qa
