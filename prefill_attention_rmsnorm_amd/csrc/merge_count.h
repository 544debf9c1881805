// Arrival counter of the in-launch decode merge (host and device).
//
// Every workgroup of a (sequence, kv head) pair adds merge_count_add(d) to
// the pair's 32-bit counter once its partial is stored, with
// d = (XCC_ID - workgroup id) mod 8 in [0, 8).  The word packs three fields:
//   bits  0.. 6  number of arrivals          (at most 127 splits)
//   bits  7..16  sum of d                    (at most 7 * 127 = 889 < 2^10)
//   bits 17..29  sum of d^2                  (at most 49 * 127 = 6223 < 2^13)
// so no field carries into the next for n_split <= 127.  The workgroup that
// sees n_split - 1 earlier arrivals is the last one.  Its pair shared one
// XCD exactly when every d was equal: with mean m = sum(d) / n, the sum of
// squares equals n m^2 only when the variance is zero, so "sum d = n d_last
// and sum d^2 = n d_last^2" is both necessary and sufficient.
//
// A counter word left over from other use of the memory (the counter must
// be zero when a call starts) shows itself to any arriver as a value that a
// zeroed counter cannot reach before the last arrival: a count of n_split or
// more, or sums larger than 7 (resp. 49) times the count.
#pragma once

#include <hip/hip_runtime.h>

namespace qa {

constexpr int kInlineMaxSplits = 127;

__host__ __device__ constexpr unsigned merge_count_add(unsigned d) {
  return 1u | (d << 7) | ((d * d) << 17);
}

__host__ __device__ constexpr unsigned merge_count_n(unsigned w) { return w & 0x7fu; }
__host__ __device__ constexpr unsigned merge_count_dsum(unsigned w) { return (w >> 7) & 0x3ffu; }
__host__ __device__ constexpr unsigned merge_count_d2sum(unsigned w) { return w >> 17; }

// Whether `old` (the value an arriver's atomic add returned) can be reached
// from zero by fewer than n_split arrivals.
__host__ __device__ constexpr bool merge_count_valid(unsigned old, unsigned n_split) {
  return merge_count_n(old) < n_split && merge_count_dsum(old) <= 7u * merge_count_n(old) &&
         merge_count_d2sum(old) <= 49u * merge_count_n(old);
}

// Whether the arriver that saw `old` is the last of n_split.
__host__ __device__ constexpr bool merge_count_last(unsigned old, unsigned n_split) {
  return merge_count_n(old) == n_split - 1u;
}

// For the last arriver (own offset d, final word total): whether all n_split
// arrivals had the same offset, i.e. ran on one XCD.
__host__ __device__ constexpr bool merge_count_one_xcd(unsigned total, unsigned n_split,
                                                       unsigned d) {
  return merge_count_dsum(total) == n_split * d && merge_count_d2sum(total) == n_split * d * d;
}

}  // namespace qa
