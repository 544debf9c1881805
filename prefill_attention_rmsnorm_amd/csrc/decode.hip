// Single-token decode on gfx950: split-K over the cache, memory-bound.
//
// "dryft-flash-infer" agent guide, Where the wins are: per-step overhead and
// the preallocated, strided cache.  A workgroup owns (split, kv head,
// sequence).  The cache rows before the new position are cut into near-equal
// runs, one per split workgroup: it first issues all of its cache loads with
// 16-byte loads, then, while they are in flight, forms q' for the G query
// heads of the group.  Scores are a 16x16x32 bf16 MFMA (heads x keys, K
// loaded straight into the B-operand layout); the softmax weights of key
// pairs are packed as bf16x2 so P.V runs on dot2 instructions over the V rows
// as loaded.  The four key groups of a wave are summed with lane swaps, the
// four waves through LDS, and the workgroup writes a partial (max, sum,
// unnormalised output).  One more workgroup per (sequence, kv head) handles
// the new token alone: the K prologue (fp64, one RNE), the cache write, and
// the one-key partial of the new slot.  It reads no cache rows and so runs
// beside the streaming workgroups instead of lengthening one of them.
//
// When the pairs fill whole rounds of the 8-XCD deal (a.sync set), the
// partials are merged inside the launch.  Workgroups are dealt to the XCDs
// round-robin by id, so the grid is numbered to give all of a pair's
// workgroups one id residue mod 8, hence one XCD: their partials meet in that
// XCD's L2.  Each workgroup stores its partial, waits for the stores and
// counts itself in on the pair's counter with a device-scope atomic; the last
// one checks from the counter that the pair really shared an XCD, drops its
// L1, reads the partials from L2, merges them in split order (the same
// arithmetic as merge.hip) and returns the counter to zero.  Otherwise
// merge.hip runs as a second launch.
#include <utility>

#include "qa.h"
#include "qa_device.h"

namespace qa {

// Sum over the four 16-lane rows of a wave of N values per lane (N a multiple
// of 4).  On return lane l holds N/4 sums: entry j is the sum of input
// 4j + 2*((l >> 4) & 1) + ((l >> 5) & 1).  A 32-lane swap pairs inputs 2j and
// 2j+1 so that lanes 0-31 add the two halves of one and lanes 32-63 of the
// other; a 16-lane swap does the same between neighbouring rows.
template <int N>
__device__ __forceinline__ void rows4_sum(const float (&v)[N], float (&r)[N / 4]) {
  float h[N / 2];
#pragma unroll
  for (int j = 0; j < N / 2; ++j) {
    const auto t = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[2 * j]),
                                                    __float_as_uint(v[2 * j + 1]),
                                                    false, false);
    h[j] = __uint_as_float(t[0]) + __uint_as_float(t[1]);
  }
#pragma unroll
  for (int j = 0; j < N / 4; ++j) {
    const auto t = __builtin_amdgcn_permlane16_swap(__float_as_uint(h[2 * j]),
                                                    __float_as_uint(h[2 * j + 1]),
                                                    false, false);
    r[j] = __uint_as_float(t[0]) + __uint_as_float(t[1]);
  }
}

// Loads of the raw q rows of the heads w, w+4, ... of the group (elements
// lane and lane+64), the norm weights and the rotation frequency of pair
// `lane`.  Issued before any cache row, since the memory counter is waited on
// in issue order.
template <int G>
struct QRaw {
  static constexpr int HPW = (G + 3) / 4;  // query heads per wave
  uint16_t x0[HPW], x1[HPW];
  uint16_t w0, w1;
  double invf;
  __device__ __forceinline__ void load(const DecodeArgs& a, const RopeFreq& f, int b,
                                       int g, int w, int lane) {
    invf = f.inv_freq[lane];  // (a lane-indexed kernel-argument load)
#pragma unroll
    for (int i = 0; i < HPW; ++i) {
      const int hl = min(w + 4 * i, G - 1);
      const uint16_t* qr = a.q + ((size_t)b * a.n_q_heads + g * G + hl) * kHeadDim;
      x0[i] = qr[lane];
      x1[i] = qr[lane + 64];
    }
    // loaded from a valid address whether or not weights are given, so no
    // branch sits between the loads
    const uint16_t* wp = a.q_norm_w ? a.q_norm_w : a.q;
    w0 = wp[lane];
    w1 = wp[lane + 64];
  }
  // q' = RoPE(RMSNorm(q) * w) * scale * log2(e), rounded to bf16 into s_q.
  __device__ __forceinline__ void compute(const DecodeArgs& a, int pos, int w, int lane,
                                          uint16_t (*s_q)[kHeadDim]) const {
    float s32, c32;
    sincos_reduced((double)pos * invf, &s32, &c32);
    const float wf0 = a.q_norm_w ? bf_to_f(w0) : 1.f;
    const float wf1 = a.q_norm_w ? bf_to_f(w1) : 1.f;
#pragma unroll
    for (int i = 0; i < HPW; ++i) {
      const int hl = w + 4 * i;
      if (hl >= G) break;
      const float y0f = bf_to_f(x0[i]), y1f = bf_to_f(x1[i]);
      const float ss = wave_sum(y0f * y0f + y1f * y1f);
      const float rinv = 1.0f / sqrtf(ss * (1.0f / 128.0f) + (float)a.eps);
      const float y0 = y0f * rinv * wf0, y1 = y1f * rinv * wf1;
      const uint32_t pk = pack_bf16x2((y0 * c32 - y1 * s32) * a.qscale,
                                      (y1 * c32 + y0 * s32) * a.qscale);
      s_q[hl][lane] = (uint16_t)(pk & 0xffffu);
      s_q[hl][lane + 64] = (uint16_t)(pk >> 16);
    }
  }
};

// The new token of sequence b, kv head g: k' (fp64, one RNE) and v written to
// slot pos, and per query head the partial of that one key: m = q'.k',
// l = 1, o = v.
template <int G>
__device__ __forceinline__ void new_token(const DecodeArgs& a, const RopeFreq& f, int b,
                                          int g, int pos, bool ok, size_t rowbase,
                                          uint16_t (*s_q)[kHeadDim], float* s_knew) {
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  if (!ok) {  // an invalid position writes nothing to the cache
    if (tid < G) {
      a.part_m[rowbase + tid] = -__builtin_inff();
      a.part_l[rowbase + tid] = 0.f;
    }
    return;
  }
  const size_t pairidx = (size_t)b * a.n_kv_heads + g;
  QRaw<G> qr;
  qr.load(a, f, b, g, w, lane);
  const uint16_t* kwp = a.k_norm_w ? a.k_norm_w : a.q;
  const uint16_t kw0r = kwp[lane], kw1r = kwp[lane + 64];
  const uint16_t* kr0 = a.k + pairidx * kHeadDim;
  const uint16_t kx0 = kr0[lane], kx1 = kr0[lane + 64];
  const uint32_t vx = reinterpret_cast<const uint32_t*>(a.v + pairidx * kHeadDim)[lane];
  if (w == 0) {
    double sn, cn;
    sincos((double)pos * qr.invf, &sn, &cn);
    uint16_t o0, o1;
    const double wk0 = a.k_norm_w ? (double)bf_to_f(kw0r) : 1.0;
    const double wk1 = a.k_norm_w ? (double)bf_to_f(kw1r) : 1.0;
    kprime_pair(kx0, kx1, wk0, wk1, a.eps, cn, sn, &o0, &o1);
    const size_t crow = (size_t)b * a.c.sb + (size_t)g * a.c.sh + (size_t)pos * a.c.sp;
    a.c.k[crow + lane] = o0;
    a.c.k[crow + lane + 64] = o1;
    reinterpret_cast<uint32_t*>(a.c.v + crow)[lane] = vx;
    s_knew[lane] = bf_to_f(o0);
    s_knew[lane + 64] = bf_to_f(o1);
  }
  qr.compute(a, pos, w, lane, s_q);
  __syncthreads();
  for (int hl = w; hl < G; hl += 4) {
    float d = bf_to_f(s_q[hl][lane]) * s_knew[lane] +
              bf_to_f(s_q[hl][lane + 64]) * s_knew[lane + 64];
    d = wave_sum(d);
    *reinterpret_cast<float2*>(a.part_o + (rowbase + hl) * kHeadDim + 2 * lane) =
        make_float2(bf_lo(vx), bf_hi(vx));
    if (lane == 0) {
      a.part_m[rowbase + hl] = d;
      a.part_l[rowbase + hl] = 1.f;
    }
  }
}

// Buffer loads with sc0 miss the CU's L1 and are served by the XCD's L2,
// where the other workgroups' stores of this launch have landed.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t l2_rsrc(const void* base, size_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes,
                                           0x00020000);
}

// Called by every workgroup of the pair once its partial is stored.  Each
// adds merge_count_add(d) to the pair's counter, d = (XCC_ID - id) mod 8:
// the deal may start at any XCD, but a pair's workgroups share an XCD
// exactly when they share d (merge_count.h).  A pair failing that is not
// merged: its rows are zeroed and QA_DEVERR_MERGE is set.  An arriver that
// finds a counter value no zeroed counter can reach (memory the counter
// shares with other use, not cleared by qa_workspace_init) sets
// QA_DEVERR_MERGE too; that pair's rows are then undefined.
template <int G>
__device__ __forceinline__ void merge_in_launch(const DecodeArgs& a, int pair, int b, int g) {
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
  if (!s_last) return;
  asm volatile("buffer_inv sc0" ::: "memory");  // drop this CU's L1 lines
  const bool bad = s_bad;
  if (tid == 0) {
    __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (bad) flag_error(a.err, QA_DEVERR_MERGE);
  }
  if (tid >= G * 32) return;
  const int hl = tid >> 5, d4 = (tid & 31) * 4;
  const size_t nrow = (size_t)ns * G;
  const __amdgpu_buffer_rsrc_t rm = l2_rsrc(a.part_m + (size_t)pair * nrow, nrow * 4);
  const __amdgpu_buffer_rsrc_t rl = l2_rsrc(a.part_l + (size_t)pair * nrow, nrow * 4);
  const __amdgpu_buffer_rsrc_t ro =
      l2_rsrc(a.part_o + (size_t)pair * nrow * kHeadDim, nrow * kHeadDim * 4);
  const MergeOut mo = merge_splits<32>((int)ns, [&](int s, float& m, float& l, float4& o) {
    const int row = s * G + hl;
    m = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rm, row * 4, 0, 1));
    l = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rl, row * 4, 0, 1));
    const auto o4 = __builtin_amdgcn_raw_buffer_load_b128(ro, (row * kHeadDim + d4) * 4, 0, 1);
    o = make_float4(__uint_as_float(o4[0]), __uint_as_float(o4[1]), __uint_as_float(o4[2]),
                    __uint_as_float(o4[3]));
  });
  const size_t hrow = (size_t)b * a.n_q_heads + g * G + hl;
  store_merged(mo, bad, a.out + hrow * kHeadDim + d4, a.lse && d4 == 0 ? a.lse + hrow : nullptr);
}

// NT: 16-key tiles per split.  Tiles are scored in pairs (2m, 2m+1) so the
// weights of keys k and k+16 pack into one bf16x2; wave w scores pairs
// w, w+4, ...  Thread (kg, c) holds V rows kg + 16i (i < NT), dims 8c..8c+7.
// Splits 0 .. n_split-2 stream the cache; split n_split-1 is the new token.
template <int G, int NT>
__global__ __launch_bounds__(256) void decode_kernel(DecodeArgs a, RopeFreq f) {
  constexpr int NP = (NT + 1) / 2;  // tile pairs
  constexpr int PW = (NP + 3) / 4;  // tile pairs per wave (at most)
  static_assert(NT >= 1 && NT <= kDecodeMaxTiles, "split length");
  static_assert(G <= 8, "group");
  __shared__ __attribute__((aligned(16))) uint16_t s_q[G][kHeadDim];
  __shared__ float s_max[4][8];
  __shared__ float s_sum[4][8];
  __shared__ __attribute__((aligned(16))) uint32_t s_pp[NP][16][8];
  __shared__ __attribute__((aligned(16))) float s_red[4][G][kHeadDim];

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  // One-dimensional grid: the cache splits of every pair first, then the
  // new-token workgroups, so the streaming workgroups are dealt out to the
  // CUs evenly and the small ones fill in behind them.  With the in-launch
  // merge, id 8 * (split * npair / 8 + k) + x is split `split` of pair
  // x + 8k, so a pair's workgroups share id mod 8.
  const int nc = a.n_split - 1;  // cache splits
  const int npair = a.batch * a.n_kv_heads;
  const int bid = blockIdx.x;
  int pair, split;
  if (a.sync) {
    const int ppx = npair >> 3, idx = bid >> 3;
    split = idx / ppx;
    pair = (bid & 7) + 8 * (idx - split * ppx);
  } else if (bid < npair * nc) {
    pair = bid / nc;
    split = bid - pair * nc;
  } else {
    pair = bid - npair * nc;
    split = nc;
  }
  const int b = pair / a.n_kv_heads, g = pair - b * a.n_kv_heads;
  const int pos = a.positions[b];
  const bool ok = pos >= 0 && pos < a.max_ctx;
  if (!ok && split == 0 && g == 0 && tid == 0)
    flag_error(a.err, QA_DEVERR_POSITION);
  const size_t pairidx = (size_t)pair;
  const size_t rowbase = (pairidx * a.n_split + split) * G;
  const float ninf = -__builtin_inff();
  do {  // every path ends at the merge below
  if (split == nc) {
    new_token<G>(a, f, b, g, pos, ok, rowbase, s_q, &s_red[0][0][0]);
    break;
  }
  // Cache rows [0, pos) -- everything before the new slot -- in nc
  // near-equal runs, so every workgroup streams the same number of rows
  // whatever the position; a run is at most ceil((max_ctx - 1) / nc) <= 16 NT
  // rows (checked at launch).
  const int nrows = ok ? pos : 0;
  const int k0 = (int)((long)split * nrows / nc);
  const int k1 = (int)((long)(split + 1) * nrows / nc);
  if (k0 >= k1) {  // nothing to attend in this split
    if (tid < G) {
      a.part_m[rowbase + tid] = ninf;
      a.part_l[rowbase + tid] = 0.f;
    }
    break;
  }
  const uint16_t* kbase = a.c.k + (size_t)b * a.c.sb + (size_t)g * a.c.sh;
  const uint16_t* vbase = a.c.v + (size_t)b * a.c.sb + (size_t)g * a.c.sh;

  // ---- 1. loads: the prologue's inputs first, then the cache rows.
  QRaw<G> qr;
  qr.load(a, f, b, g, w, lane);
  __builtin_amdgcn_sched_barrier(0);  // the small loads stay first
  // Rows past k1 are clamped to k1-1 (read again, their scores masked).
  const int klast = k1 - 1;
  // K, in the B-operand layout of the 16x16x32 MFMA: for tile t, lane l
  // holds dims 32*ks + 8*(l/16) .. +7 of key 16*t + l%16.  Pairs past the
  // split are skipped (a uniform branch); the odd tile past an odd NT is
  // loaded clamped and its scores masked.
  u32x4 kq[PW][2][4];
#pragma unroll
  for (int i = 0; i < PW; ++i) {
    const int m = w + 4 * i;
    if ((i == 0 && NP >= 4) || m < NP) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int key = min(k0 + 32 * m + 16 * j + (lane & 15), klast);
        const uint16_t* kr = kbase + (size_t)key * a.c.sp + 8 * (lane >> 4);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) kq[i][j][ks] = ld16(kr + 32 * ks);
      }
    }
  }
  // V, for every thread: 8 dims (chunk c) of keys kg + 16*i.
  const int kg = tid >> 4, c = tid & 15;
  u32x4 vr[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    const int key = min(k0 + kg + 16 * i, klast);
    vr[i] = ld16(vbase + (size_t)key * a.c.sp + 8 * c);
  }
  // keep the loads in this order, ahead of the prologue arithmetic
  __builtin_amdgcn_sched_barrier(0);

  // ---- 2. q' while the cache loads are in flight
  qr.compute(a, pos, w, lane, s_q);
  __syncthreads();

  // ---- 3. scores.  Wave w forms S = q' K^T for its tile pairs with the
  // heads on the MFMA row axis: lane l holds head 4*(l/16) + r of key l%16.
  const int hrow = 4 * (lane >> 4);  // first head of this lane's registers
  f32x4 sj[PW][2];
  {
    const int qh = min(lane & 15, G - 1);
    const bool qvalid = (lane & 15) < G;
    u32x4 qv[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      qv[ks] = ld16(&s_q[qh][32 * ks + 8 * (lane >> 4)]);
      if (!qvalid) qv[ks] = u32x4{0u, 0u, 0u, 0u};
    }
    float mx[4] = {ninf, ninf, ninf, ninf};
#pragma unroll
    for (int i = 0; i < PW; ++i) {
      const int m = w + 4 * i;
      if ((i == 0 && NP >= 4) || m < NP) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          sj[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < 4; ++ks)
            sj[i][j] = mfma16x16x32(qv[ks], kq[i][j][ks], sj[i][j]);
          const bool kok = k0 + 32 * m + 16 * j + (lane & 15) < k1;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            if (!kok || hrow + r >= G) sj[i][j][r] = ninf;
            mx[r] = fmaxf(mx[r], sj[i][j][r]);
          }
        }
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float t = row16_max(mx[r]);
      if ((lane & 15) == 0 && hrow + r < G) s_max[w][hrow + r] = t;
    }
  }
  __syncthreads();

  // ---- 4. softmax weights: p = exp2(s - M) with M the split's max per head.
  // Keys (k, k+16) of a tile pair are packed as bf16x2 for the P.V dot
  // products.
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int h = min(hrow + r, G - 1);
    const float mh = fmaxf(fmaxf(s_max[0][h], s_max[1][h]), fmaxf(s_max[2][h], s_max[3][h]));
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < PW; ++i) {
      const int m = w + 4 * i;
      if ((i == 0 && NP >= 4) || m < NP) {
        const float p0 = __builtin_amdgcn_exp2f(sj[i][0][r] - mh);
        const float p1 = __builtin_amdgcn_exp2f(sj[i][1][r] - mh);
        sum += p0 + p1;
        if (hrow + r < G) s_pp[m][lane & 15][hrow + r] = pack_bf16x2(p0, p1);
      }
    }
    sum = row16_sum(sum);
    if ((lane & 15) == 0 && hrow + r < G) s_sum[w][hrow + r] = sum;
  }
  __syncthreads();

  // ---- 5. O += P.V: thread (kg, c) over its key pairs (kg + 32m, kg + 32m + 16)
  float acc[G * 8];
#pragma unroll
  for (int n = 0; n < G * 8; ++n) acc[n] = 0.f;
#pragma unroll
  for (int m = 0; m < NP; ++m) {
    uint32_t pp[G];
#pragma unroll
    for (int hl = 0; hl < G; ++hl) pp[hl] = s_pp[m][kg][hl];
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) {
      const uint32_t va = vr[2 * m][e2];
      const uint32_t vb2 = 2 * m + 1 < NT ? vr[2 * m + 1 < NT ? 2 * m + 1 : 0][e2] : 0u;
      const uint32_t lo = (va & 0xffffu) | (vb2 << 16);
      const uint32_t hi = (va >> 16) | (vb2 & 0xffff0000u);
#pragma unroll
      for (int hl = 0; hl < G; ++hl) {
        acc[8 * hl + 2 * e2] = dot2_bf16(pp[hl], lo, acc[8 * hl + 2 * e2]);
        acc[8 * hl + 2 * e2 + 1] = dot2_bf16(pp[hl], hi, acc[8 * hl + 2 * e2 + 1]);
      }
    }
  }
  // the wave's four key groups, then the four waves
  {
    float red[2 * G];
    rows4_sum<G * 8>(acc, red);
    const int s16 = (lane >> 4) & 1, s32 = (lane >> 5) & 1;
#pragma unroll
    for (int j = 0; j < 2 * G; ++j)
      s_red[w][j >> 1][8 * c + 4 * (j & 1) + 2 * s16 + s32] = red[j];
  }
  __syncthreads();

  // ---- 6. the split's partial
  if (tid < G * 32) {
    const int hl = tid >> 5, d4 = (tid & 31) * 4;
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      const float4 t = *reinterpret_cast<const float4*>(&s_red[ww][hl][d4]);
      o.x += t.x; o.y += t.y; o.z += t.z; o.w += t.w;
    }
    *reinterpret_cast<float4*>(a.part_o + (rowbase + hl) * kHeadDim + d4) = o;
    if ((tid & 31) == 0) {
      a.part_m[rowbase + hl] =
          fmaxf(fmaxf(s_max[0][hl], s_max[1][hl]), fmaxf(s_max[2][hl], s_max[3][hl]));
      a.part_l[rowbase + hl] = (s_sum[0][hl] + s_sum[1][hl]) + (s_sum[2][hl] + s_sum[3][hl]);
    }
  }
  } while (0);
  if (a.sync) merge_in_launch<G>(a, pair, b, g);
}

template <int G, int NT>
static void launch_nt(const DecodeArgs& a, const RopeFreq& f, hipStream_t s) {
  const dim3 grid(a.n_split * a.n_kv_heads * a.batch);
  hipLaunchKernelGGL((decode_kernel<G, NT>), grid, dim3(256), 0, s, a, f);
}

template <int G, int... NT>
static hipError_t launch_decode_g(const DecodeArgs& a, const RopeFreq& f,
                                  hipStream_t s, std::integer_sequence<int, NT...>) {
  const int nt = a.keys_per_split / 16;
  if (a.keys_per_split % 16 != 0 || nt < 1 || nt > kDecodeMaxTiles || a.n_split < 2 ||
      (long)(a.n_split - 1) * a.keys_per_split < a.max_ctx - 1)
    return hipErrorInvalidValue;
  ((nt == NT + 1 ? launch_nt<G, NT + 1>(a, f, s) : void()), ...);
  return hipGetLastError();
}

using kTiles = std::make_integer_sequence<int, kDecodeMaxTiles>;

hipError_t launch_decode(const DecodeArgs& a, const RopeFreq& f, int group,
                         hipStream_t s, int* n_kernels) {
  *n_kernels = 0;
  if (a.sync && ((a.batch * a.n_kv_heads) % 8 != 0 || a.n_split > kInlineMaxSplits))
    return hipErrorInvalidValue;  // the grid numbering and the counter fields
  hipError_t e;
  switch (group) {
    case 1: e = launch_decode_g<1>(a, f, s, kTiles{}); break;
    case 2: e = launch_decode_g<2>(a, f, s, kTiles{}); break;
    case 4: e = launch_decode_g<4>(a, f, s, kTiles{}); break;
    case 8: e = launch_decode_g<8>(a, f, s, kTiles{}); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  *n_kernels = 1;
  if (a.sync) return hipSuccess;  // merged inside the launch
  e = launch_merge(a, group, s);
  if (e == hipSuccess) *n_kernels = 2;
  return e;
}

}  // namespace qa
