// Verification of a speculative draft block on gfx950.
//
// "dryft-flash-infer" agent guide, Where the wins are: speculative decoding
// with exact verification reproduces the greedy argmax, so the block's rows
// must equal what sequential decode steps would give.  The draft's
// block_len tokens x G heads of one KV head form up to 128 query rows that
// share every K/V tile (MFMA tile machinery of the prefill kernel); the keys
// are split across workgroups, each writing a partial that merge.hip
// combines in split order.
//
// Splits 0 .. n_split-2 take near-equal runs of whole 64-key tiles of the
// slots before the block (cut on the device from the start position, so the
// grid depends on the launch sizes only); split n_split-1 runs the prologue
// for the block's own slots (k' in fp64 with one RNE), writes them to the
// cache and attends to them alone, so the prologue, the longest part of any
// workgroup's start, is not followed by a long run of cache tiles.  Only
// that workgroup ever reads the block's slots in this call, and the block
// barrier orders its own writes before its reads.
#include "attn_tile.h"
#include "qa.h"
#include "verify_layout.h"

namespace qa {

// Byte offset of the (cos, sin) of rotation pair i for draft token t in the
// LDS table the query prologue reads (QPrologue::cs_from_lds): 512-byte rows,
// 16-byte chunk c = i / 2 of row t at chunk position c ^ (t & 31).
__device__ __forceinline__ uint32_t cs_lds_offset(int t, int i) {
  return (uint32_t)(t * 512 + (((i >> 1) ^ (t & 31)) << 4) + ((i & 1) << 3));
}

// RING: the old-slot splits stream their tiles through the four-stage ring
// of attn_tile.h (2 or 4 waves, blocks of up to kVerifyRingTokens tokens);
// the block's own split, one tile long, takes the double-buffered pass over
// the ring's first buffers.
template <int G, int NW, bool RING>
__global__ __launch_bounds__(NW * 64) void verify_kernel(DecodeArgs a, RopeFreq f) {
  constexpr int NT = NW * 64;
  // cos/sin rows of the block's tokens: up to 128/G, or kVerifyRingTokens
  constexpr int kCsBytes = (RING ? kVerifyRingTokens : 128 / G) * 512;
  constexpr int kRingBytes = RING ? kKTileBytes : 16;
  __shared__ __attribute__((aligned(16))) unsigned char lds_k0[kKTileBytes];
  __shared__ __attribute__((aligned(16))) unsigned char lds_k1[kKTileBytes];
  __shared__ __attribute__((aligned(16))) unsigned char lds_v0[kKTileBytes];
  // Without the ring, V tile 1 and the queries' cos/sin rows share one
  // array: the rows are read by the query prologue, which every wave
  // finishes before the first barrier of attend(), and V tile 1 is first
  // copied in after that barrier.  With it, the rows have their own array,
  // since the ring's copies start before the prologue.
  __shared__ __attribute__((aligned(16)))
  unsigned char lds_v1[!RING && kCsBytes > kKTileBytes ? kCsBytes : kKTileBytes];
  __shared__ __attribute__((aligned(16))) unsigned char lds_k2[kRingBytes];
  __shared__ __attribute__((aligned(16))) unsigned char lds_k3[kRingBytes];
  __shared__ __attribute__((aligned(16))) unsigned char lds_v2[kRingBytes];
  __shared__ __attribute__((aligned(16))) unsigned char lds_v3[kRingBytes];
  __shared__ __attribute__((aligned(16))) unsigned char lds_csr[RING ? kCsBytes : 16];
  (void)lds_csr;
  const AttnLds lds{lds_k0, lds_k1, lds_v0, lds_v1};
  const RingLds ring{lds_k0, lds_k1, lds_k2, lds_k3, lds_v0, lds_v1, lds_v2, lds_v3};
  unsigned char* lds_cs = RING ? lds_csr : lds_v1;

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int j = l & 31, h2 = l >> 5;
  // One-dimensional grid, a pair's splits contiguous.
  const int pair = blockIdx.x / a.n_split, split = blockIdx.x - pair * a.n_split;
  const int b = pair / a.n_kv_heads, g = pair - b * a.n_kv_heads;
  const int n = a.block_len;
  const int rows = n * G;
  const int n_old = a.n_split - 1;
  const bool new_split = split == n_old;
  const int r = 32 * w + j;
  const bool row_ok = r < rows;
  const int hl = row_ok ? r / n : 0, ti = row_ok ? r % n : 0;
  const int h = g * G + hl;

  // ---- loads that do not depend on the block's position go out first: the
  // query row and its norm weights, and for the new slots' workgroup the
  // first round of the block's k/v rows (token i = w + NW c of the block)
  constexpr int CH = 8;  // new slots per round and wave
  const int L0 = a.positions[b];
  QPrologue qp;
  qp.load_qw(a.q + (((size_t)b * n + ti) * a.n_q_heads + h) * kHeadDim, row_ok, a.q_norm_w,
             h2);
  uint16_t kx0[CH], kx1[CH];
  uint32_t vx[CH];
  double wk0 = 1.0, wk1 = 1.0, invf = 0.0;
  if (new_split) {
    invf = f.inv_freq[l];
    if (a.k_norm_w) {
      wk0 = (double)bf_to_f(a.k_norm_w[l]);
      wk1 = (double)bf_to_f(a.k_norm_w[l + 64]);
    }
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int i = min(w + NW * c, n - 1);
      const size_t src = (((size_t)b * n + i) * a.n_kv_heads + g) * kHeadDim;
      kx0[c] = a.k[src + l];
      kx1[c] = a.k[src + l + 64];
      vx[c] = reinterpret_cast<const uint32_t*>(a.v + src)[l];
    }
  }

  const bool ok = L0 >= 0 && L0 + n <= a.max_ctx;
  if (!ok && split == 0 && g == 0 && tid == 0) flag_error(a.err, QA_DEVERR_POSITION);
  int k0, k1;
  if (!new_split) {  // tiles t0 .. t1-1 of the slots before the block
    const int nt = ok ? (L0 + kKeyTile - 1) / kKeyTile : 0;
    const int t0 = (int)((long)split * nt / n_old);
    const int t1 = (int)((long)(split + 1) * nt / n_old);
    k0 = t0 * kKeyTile;
    k1 = ok ? min(t1 * kKeyTile, L0) : 0;
  } else {  // the block's own slots
    k0 = ok ? L0 : 0;
    k1 = ok ? L0 + n : 0;
  }
  const size_t pairidx = (size_t)b * a.n_kv_heads + g;
  const size_t rowbase = (pairidx * a.n_split + split) * rows;
  const int p = L0 + ti;

  if (k0 < k1) {
    const uint16_t* kbase = a.c.k + (size_t)b * a.c.sb + (size_t)g * a.c.sh;
    const uint16_t* vbase = a.c.v + (size_t)b * a.c.sb + (size_t)g * a.c.sh;
    TileLoader<NW> ld;
    ld.init(__builtin_amdgcn_readfirstlane(w), l, a.c.sp);
    // the queries' rotation frequency (the cos/sin loop below gives thread
    // tid pair tid % 64 every time), loaded ahead of the ring's copies: the
    // memory counter is in order, so a load behind them would wait for them
    const double invf_cs = f.inv_freq[tid & (kHalf - 1)];
    WaveAttn st;
    st.init(l);
    u32x4 qb[8];
    const int lim_abs = row_ok ? min(p, k1 - 1) : k1 - 1;
    // ---- cos/sin of the draft positions for the queries (LDS), one entry
    // per thread at a time: the angle reduced to whole turns in fp64, then
    // the hardware's turn-based cos/sin (the queries are rounded to bf16
    // for the MFMA, so fp32 suffices); then q'.  With copies into LDS in
    // flight the barrier orders LDS only, so that they stay in flight.
    static_assert(NT % kHalf == 0, "thread tid takes pair tid % 64");
    auto q_prologue = [&](bool copies_in_flight) {
      for (int e = tid; e < n * kHalf; e += NT) {
        const int i = e >> 6, pi = e & (kHalf - 1);
        const double turns = (double)(L0 + i) * invf_cs * 0.15915494309189535;
        const float fr = (float)(turns - floor(turns));
        *reinterpret_cast<float2*>(lds_cs + cs_lds_offset(i, pi)) =
            make_float2(__builtin_amdgcn_cosf(fr), __builtin_amdgcn_sinf(fr));
      }
      if (copies_in_flight) lds_barrier();
      else __syncthreads();
      qp.cs_from_lds(lds_cs, ti, h2);
      qp.compute((float)a.eps, a.qscale, qb);
    };
    // An old-slot split with the ring runs straight through: its copies go
    // out first, then the queries' prologue, then the tiles.  (Kept apart
    // from the other path, so that the compiler's waits for the loads before
    // the copies count the copies exactly instead of draining them.)
    bool done = false;
    if constexpr (RING) {
      if (!new_split) {
        ring_first(ld, ring, kbase, vbase, a.c.sp, k0, k1);
        q_prologue(true);
        // keys below k1 <= L0 <= every query's position: only a partial last
        // tile is masked
        attend_ring(st, ld, ring, kbase, vbase, a.c.sp, k0, k1,
                    ((k1 - k0) & (kKeyTile - 1)) != 0, qb, lim_abs, h2);
        done = true;
      }
    }
    if (!done) {
      // ---- new slots: k' (fp64) and v into the cache.  Wave w takes slots
      // L0 + w, L0 + w + NW, ...; the rotation advances from one slot to the
      // next by the fp64 angle-addition identity (one turn by NW positions)
      // instead of a fresh sincos per slot.
      if (new_split && w < n) {  // (wave-uniform)
        double cn, sn, cstep, sstep;
        sincos((double)(L0 + w) * invf, &sn, &cn);
        sincos((double)NW * invf, &sstep, &cstep);
        for (int i0 = w; i0 < n; i0 += NW * CH) {
          if (i0 != w) {  // later rounds (blocks longer than NW * CH)
  #pragma unroll
            for (int c = 0; c < CH; ++c) {
              const int i = min(i0 + NW * c, n - 1);
              const size_t src = (((size_t)b * n + i) * a.n_kv_heads + g) * kHeadDim;
              kx0[c] = a.k[src + l];
              kx1[c] = a.k[src + l + 64];
              vx[c] = reinterpret_cast<const uint32_t*>(a.v + src)[l];
            }
          }
          // The slots' sums of squares are reduced across the wave together,
          // one butterfly step for all of them at a time, so their shuffle
          // latencies overlap.  Per slot the arithmetic is kprime_pair's: the
          // same products and sums in the same order.
          double ss[CH];
          {
  #pragma clang fp contract(off)
  #pragma unroll
            for (int c = 0; c < CH; ++c) {
              const double x0 = (double)bf_to_f(kx0[c]), x1 = (double)bf_to_f(kx1[c]);
              ss[c] = x0 * x0 + x1 * x1;
            }
  #pragma unroll
            for (int o = 32; o >= 1; o >>= 1)
  #pragma unroll
              for (int c = 0; c < CH; ++c) ss[c] += __shfl_xor(ss[c], o);
          }
  #pragma unroll
          for (int c = 0; c < CH; ++c) {
            const int i = i0 + NW * c;
            if (i >= n) break;  // (wave-uniform)
            uint16_t o0, o1;
            {
  #pragma clang fp contract(off)
              const double x0 = (double)bf_to_f(kx0[c]), x1 = (double)bf_to_f(kx1[c]);
              const double rr = sqrt(ss[c] / 128.0 + a.eps);
              const double y0 = x0 / rr * wk0;
              const double y1 = x1 / rr * wk1;
              o0 = f64_to_bf16_rne(y0 * cn - y1 * sn);
              o1 = f64_to_bf16_rne(y1 * cn + y0 * sn);
            }
            const size_t crow =
                (size_t)b * a.c.sb + (size_t)g * a.c.sh + (size_t)(L0 + i) * a.c.sp;
            a.c.k[crow + l] = o0;
            a.c.k[crow + l + 64] = o1;
            reinterpret_cast<uint32_t*>(a.c.v + crow)[l] = vx[c];
            const double c2 = cn * cstep - sn * sstep;
            sn = sn * cstep + cn * sstep;
            cn = c2;
          }
        }
      }
      q_prologue(false);
      // cache slots written by earlier calls: their first tiles load now,
      // with q' already formed, so nothing but the copies stands before the
      // first tile; the new slots' workgroup first orders its own cache writes
      if (!new_split) load_first(ld, lds, kbase, vbase, a.c.sp, k0, k1);
      __syncthreads();
      if (new_split) load_first(ld, lds, kbase, vbase, a.c.sp, k0, k1);
      // tiles whose keys all lie below k1 and at or below the first draft
      // position need no mask
      const int n_unmasked = max(min(k1 - 1, L0) + 1 - k0, 0) / kKeyTile;
      attend(st, ld, lds, kbase, vbase, a.c.sp, k0, k1, n_unmasked, qb, lim_abs, h2);
    }
    if (row_ok) {
      const float lt = st.lsum + __shfl_xor(st.lsum, 32);
      if (h2 == 0) {
        a.part_m[rowbase + r] = st.m;
        a.part_l[rowbase + r] = lt;
      }
      float* po = a.part_o + (rowbase + r) * kHeadDim;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          // non-temporal: the partials are read once, by the merge kernel on
          // whichever XCD, so they need not stay in this XCD's L2
          const f32x4 v4 = {st.o[db][4 * a4], st.o[db][4 * a4 + 1], st.o[db][4 * a4 + 2],
                            st.o[db][4 * a4 + 3]};
          __builtin_nontemporal_store(v4, reinterpret_cast<f32x4*>(po + 32 * db + 8 * a4 + 4 * h2));
        }
    }
  } else {
    for (int rr = tid; rr < rows; rr += NT) {
      a.part_m[rowbase + rr] = -__builtin_inff();
      a.part_l[rowbase + rr] = 0.f;
    }
  }
}

template <int G>
static hipError_t launch_verify_g(const DecodeArgs& a, const RopeFreq& f,
                                  hipStream_t s) {
  const dim3 grid(a.n_split * a.n_kv_heads * a.batch);
  const int rows = a.block_len * G;
  const bool ring = verify_uses_ring(G, a.block_len);
  if (rows <= 32)
    hipLaunchKernelGGL((verify_kernel<G, 1, false>), grid, dim3(64), 0, s, a, f);
  else if (rows <= 64 && ring)
    hipLaunchKernelGGL((verify_kernel<G, 2, true>), grid, dim3(128), 0, s, a, f);
  else if (rows <= 64)
    hipLaunchKernelGGL((verify_kernel<G, 2, false>), grid, dim3(128), 0, s, a, f);
  else if (rows <= 128 && ring)
    hipLaunchKernelGGL((verify_kernel<G, 4, true>), grid, dim3(256), 0, s, a, f);
  else if (rows <= 128)
    hipLaunchKernelGGL((verify_kernel<G, 4, false>), grid, dim3(256), 0, s, a, f);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_verify(const DecodeArgs& a, const RopeFreq& f, int group,
                         hipStream_t s, int* n_kernels) {
  *n_kernels = 0;
  if (a.sync) return hipErrorInvalidValue;  // verify partials merge in their own launch
  hipError_t e;
  switch (group) {
    case 1: e = launch_verify_g<1>(a, f, s); break;
    case 2: e = launch_verify_g<2>(a, f, s); break;
    case 4: e = launch_verify_g<4>(a, f, s); break;
    case 8: e = launch_verify_g<8>(a, f, s); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  *n_kernels = 1;
  e = launch_merge(a, group, s);
  if (e == hipSuccess) *n_kernels = 2;
  return e;
}

}  // namespace qa
