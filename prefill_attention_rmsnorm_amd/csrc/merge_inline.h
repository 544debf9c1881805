// Split-K partials merged inside the launch that wrote them (decode),
// through one XCD's L2.
//
// Workgroups are dealt to the XCDs round-robin by id, so a grid numbered to
// give all of a (sequence, kv head) pair's workgroups one id residue mod 8
// keeps the pair on one XCD, and their partials meet in that XCD's L2.  Each
// workgroup stores its partial, waits for the stores and counts itself in on
// the pair's counter with a device-scope atomic; the last one checks from the
// counter that the pair really shared an XCD, drops its L1, reads the
// partials from L2, merges them in split order (merge_splits_n in batches of
// 8 splits; merge.hip takes the same single batch up to 8 splits, so the two
// paths agree bit for bit there, and one batch of 16 above that) and returns
// the counter to zero.
#pragma once

#include "qa.h"
#include "qa_device.h"

namespace qa {

// Buffer loads with sc0 miss the CU's L1 and are served by the XCD's L2,
// where the other workgroups' stores of this launch have landed.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t l2_rsrc(const void* base, size_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes,
                                           0x00020000);
}

// Called by every workgroup of the pair (all threads) once its partial is
// stored.  Each adds merge_count_add(d) to the pair's counter,
// d = (XCC_ID - id) mod 8: the deal may start at any XCD, but a pair's
// workgroups share an XCD exactly when they share d (merge_count.h).  Returns
// true in the last workgroup; *bad then tells that the pair did not share an
// XCD (its rows are zeroed and QA_DEVERR_MERGE is set).  An arriver that finds
// a counter value no zeroed counter can reach (memory the counter shares with
// other use, not cleared by qa_workspace_init) sets QA_DEVERR_MERGE too; that
// pair's rows are then undefined.
__device__ __forceinline__ bool merge_arrive(const DecodeArgs& a, int pair, bool* bad) {
  __shared__ int s_last, s_bad;
  const int tid = threadIdx.x;
  const unsigned ns = (unsigned)a.n_split;
  unsigned* ctr = a.sync - kSyncWords * (pair + 1);
  __builtin_amdgcn_s_waitcnt(0);  // this wave's partial stores are in L2
  __syncthreads();
  if (tid == 0) {
    const unsigned d = (__builtin_amdgcn_s_getreg((3 << 11) | 20) - blockIdx.x) & 7u;
    const unsigned add = merge_count_add(d);  // HW_REG_XCC_ID above
    const unsigned old =
        __hip_atomic_fetch_add(ctr, add, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (!merge_count_valid(old, ns)) flag_error(a.err, QA_DEVERR_MERGE);
    s_last = merge_count_last(old, ns);
    s_bad = !merge_count_one_xcd(old + add, ns, d);
  }
  __syncthreads();
  *bad = s_bad;
  return s_last;
}

// The pair's merge in its last workgroup (NT threads): rows = block_len * G
// partial rows (row r is head r / block_len, draft token r % block_len),
// each as 32 groups of 4 dims; every thread takes IG (row, dims) items at a
// time with all of their loads in flight.
template <int NT, int IG>
__device__ __forceinline__ void merge_pair(const DecodeArgs& a, int pair, int b, int g, int G) {
  bool bad;
  if (!merge_arrive(a, pair, &bad)) return;
  asm volatile("buffer_inv sc0" ::: "memory");  // drop this CU's L1 lines
  const int tid = threadIdx.x;
  if (tid == 0) {
    __hip_atomic_store(a.sync - kSyncWords * (pair + 1), 0u, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
    if (bad) flag_error(a.err, QA_DEVERR_MERGE);
  }
  const int n = a.block_len, rows = n * G, items = rows * 32, ns = a.n_split;
  const size_t nrow = (size_t)ns * rows;
  const __amdgpu_buffer_rsrc_t rm = l2_rsrc(a.part_m + (size_t)pair * nrow, nrow * 4);
  const __amdgpu_buffer_rsrc_t rl = l2_rsrc(a.part_l + (size_t)pair * nrow, nrow * 4);
  const __amdgpu_buffer_rsrc_t ro =
      l2_rsrc(a.part_o + (size_t)pair * nrow * kHeadDim, nrow * kHeadDim * 4);
  for (int it0 = tid; it0 < items; it0 += NT * IG) {
    MergeOut mo[IG];
    merge_splits_n<8, IG>(
        ns,
        [&](int j, int s, float& m, float& l, float4& o) {
          const int it = min(it0 + NT * j, items - 1);
          const int row = s * rows + (it >> 5), d4 = (it & 31) * 4;
          m = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rm, row * 4, 0, 1));
          l = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rl, row * 4, 0, 1));
          const auto o4 =
              __builtin_amdgcn_raw_buffer_load_b128(ro, (row * kHeadDim + d4) * 4, 0, 1);
          o = make_float4(__uint_as_float(o4[0]), __uint_as_float(o4[1]),
                          __uint_as_float(o4[2]), __uint_as_float(o4[3]));
        },
        mo);
#pragma unroll
    for (int j = 0; j < IG; ++j) {
      const int it = it0 + NT * j;
      if (it >= items) break;
      const int r = it >> 5, d4 = (it & 31) * 4;
      const int hl = r / n, ti = r - hl * n;
      const size_t hrow = ((size_t)b * n + ti) * a.n_q_heads + g * G + hl;
      store_merged(mo[j], bad, a.out + hrow * kHeadDim + d4,
                   a.lse && d4 == 0 ? a.lse + hrow : nullptr);
    }
  }
}

}  // namespace qa
