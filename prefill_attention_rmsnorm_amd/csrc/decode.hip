// Single-token decode on gfx950: split-K over the cache, memory-bound.
//
// "dryft-flash-infer" agent guide, Where the wins are: per-step overhead and
// the preallocated, strided cache.  A workgroup of kDecodeWaves (nine) waves
// owns (split, kv head, sequence); the cache rows before the new position are
// cut into near-equal runs, one per split, and wave w owns the 16-key tiles
// w, w+9, ... of its run.  Every wave loads the small inputs (the position, the raw q
// rows of all heads of the group) and forms q' for all heads itself, so no
// wave waits for another before its first tile; its cache loads (K straight
// into the A-operand layout of the 16x16x32 bf16 MFMA, V as whole rows) run
// two tiles ahead of the tile it scores.  Both products of a tile are MFMAs
// with the heads on the column axis: the transposed scores S^T = K q'^T come
// out in exactly the layout the P.V product takes its weights in (the keys
// of the K operand are permuted to make it so), and O^T = V^T P^T takes V
// from the rows as loaded, so a tile costs a few dozen vector instructions
// and no LDS traffic.  Each wave keeps an online softmax per head (running
// max and sum, the output rescaled when the max grows); the waves'
// (max, sum, output) are combined once, after one barrier.  The new token is
// folded into split 0: its last wave runs the fp64 K prologue (one RNE) and
// writes the slot before issuing its own cache loads, and adds the new key to
// its softmax at the end.
//
// When the pairs fill whole rounds of the 8-XCD deal (a.sync set), the
// partials are merged inside the launch.  Workgroups are dealt to the XCDs
// round-robin by id, so the grid is numbered to give all of a pair's
// workgroups one id residue mod 8, hence one XCD: their partials meet in that
// XCD's L2.  Each workgroup stores its partial, waits for the stores and
// counts itself in on the pair's counter with a device-scope atomic; the last
// one checks from the counter that the pair really shared an XCD, drops its
// L1, reads the partials from L2, merges them in split order (the arithmetic
// of merge.hip) and returns the counter to zero.  Otherwise merge.hip runs
// as a second launch.
#include <utility>

#include "merge_inline.h"
#include "qa.h"
#include "qa_device.h"

namespace qa {

// The raw q rows of all G heads of the group (elements lane and lane+64 of
// each), the norm weights and the rotation frequency of pair `lane`; every
// wave forms q' for all heads itself, so no wave waits for another before
// its first tile.
template <int G>
struct QRaw {
  uint16_t x0[G], x1[G];
  uint16_t w0, w1;
  double invf;
  __device__ __forceinline__ void load(const DecodeArgs& a, const RopeFreq& f, int b,
                                       int g, int lane) {
    invf = f.inv_freq[lane];  // (a lane-indexed kernel-argument load)
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const uint16_t* qr = a.q + ((size_t)b * a.n_q_heads + g * G + h) * kHeadDim;
      x0[h] = qr[lane];
      x1[h] = qr[lane + 64];
    }
    // loaded from a valid address whether or not weights are given, so no
    // branch sits between the loads
    const uint16_t* wp = a.q_norm_w ? a.q_norm_w : a.q;
    w0 = wp[lane];
    w1 = wp[lane + 64];
  }
  // q' = RoPE(RMSNorm(q) * w) * scale * log2(e) for every head, rounded to
  // bf16 into the wave's patch sq.  The query side is rounded to bf16 for
  // the MFMA, so fp32 suffices: the angle is reduced to whole turns in fp64
  // and its cos/sin taken with the hardware's turn-based v_sin/v_cos; each
  // head's sum of squares is a DPP sum within each 16-lane row plus the four
  // row totals read from lanes 0, 16, 32, 48.
  __device__ __forceinline__ void compute(const DecodeArgs& a, int pos, int lane,
                                          uint16_t (*sq)[kHeadDim]) const {
    const double turns = (double)pos * invf * 0.15915494309189535;  // / (2 pi)
    const float fr = (float)(turns - floor(turns));
    const float s32 = __builtin_amdgcn_sinf(fr), c32 = __builtin_amdgcn_cosf(fr);
    const float wf0 = a.q_norm_w ? bf_to_f(w0) : 1.f;
    const float wf1 = a.q_norm_w ? bf_to_f(w1) : 1.f;
    float ss[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float y0f = bf_to_f(x0[h]), y1f = bf_to_f(x1[h]);
      ss[h] = row16_sum(y0f * y0f + y1f * y1f);
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float tot = (__int_as_float(__builtin_amdgcn_readlane(__float_as_int(ss[h]), 0)) +
                         __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ss[h]), 16))) +
                        (__int_as_float(__builtin_amdgcn_readlane(__float_as_int(ss[h]), 32)) +
                         __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ss[h]), 48)));
      const float y0f = bf_to_f(x0[h]), y1f = bf_to_f(x1[h]);
      const float rinv = 1.0f / sqrtf(tot * (1.0f / 128.0f) + (float)a.eps);
      const float y0 = y0f * rinv * wf0, y1 = y1f * rinv * wf1;
      const uint32_t pk = pack_bf16x2((y0 * c32 - y1 * s32) * a.qscale,
                                      (y1 * c32 + y0 * s32) * a.qscale);
      sq[h][lane] = (uint16_t)(pk & 0xffffu);
      sq[h][lane + 64] = (uint16_t)(pk >> 16);
    }
  }
};

// Every lane of the wave sees what the wave wrote to LDS before this point.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// TPW: 16-key tiles per wave (a run is at most 16 * kDecodeWaves * TPW
// rows); wave w owns the tiles w, w + kDecodeWaves, ... of its run.  SYNC:
// a.sync is set (the merge inside the launch); a compile-time choice, so that
// each instantiation carries one grid numbering and one ending (measured
// 0.18 us faster per call than deciding at run time).
template <int G, int TPW, bool SYNC>
__global__ __launch_bounds__(64 * kDecodeWaves, 2) void decode_kernel(DecodeArgs a, RopeFreq f) {
  constexpr int NW = kDecodeWaves;
  static_assert(TPW >= 1 && TPW <= 4, "tiles per wave");
  static_assert(G <= 8, "group");
  __shared__ __attribute__((aligned(16))) uint16_t s_q[NW][G][kHeadDim];
  __shared__ __attribute__((aligned(16))) float s_red[NW][G][kHeadDim];
  __shared__ float s_m[NW][G], s_l[NW][G];

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int ns = a.n_split;
  const int npair = a.batch * a.n_kv_heads;
  const int bid = blockIdx.x;
  // One-dimensional grid.  With the in-launch merge, id
  // 8 * (split * npair / 8 + k) + x is split `split` of pair x + 8k, so a
  // pair's workgroups share id mod 8; otherwise pairs are contiguous.
  int pair, split;
  if constexpr (SYNC) {
    const int ppx = npair >> 3, idx = bid >> 3;
    split = idx / ppx;
    pair = (bid & 7) + 8 * (idx - split * ppx);
  } else {
    pair = bid / ns;
    split = bid - pair * ns;
  }
  const int b = pair / a.n_kv_heads, g = pair - b * a.n_kv_heads;
  const size_t rowbase = ((size_t)pair * ns + split) * G;
  const float ninf = -__builtin_inff();
  const bool nt_wave = split == 0 && w == NW - 1;  // the new token's prologue and key
  const int kg = lane >> 4, c = lane & 15;
  uint16_t (*sq)[kHeadDim] = s_q[w];  // this wave's q'

  // ---- 1. the small loads: the position (the cache loads wait for it),
  // the q rows, and in the new token's wave its k/v row (V as dims
  // 8c .. 8c+7, the layout of the P.V step) and the k norm weights
  const int pos = a.positions[b];
  QRaw<G> qr;
  qr.load(a, f, b, g, lane);
  uint16_t nk0 = 0, nk1 = 0, nw0 = 0, nw1 = 0;
  u32x4 nv[4] = {};  // dims 32 kg + 8 r .. +7 for r < 4 (the O^T layout)
  if (nt_wave) {
    const uint16_t* kr = a.k + (size_t)pair * kHeadDim;
    nk0 = kr[lane];
    nk1 = kr[lane + 64];
    const uint16_t* kwp = a.k_norm_w ? a.k_norm_w : a.q;
    nw0 = kwp[lane];
    nw1 = kwp[lane + 64];
#pragma unroll
    for (int r = 0; r < 4; ++r) nv[r] = ld16(a.v + (size_t)pair * kHeadDim + 32 * kg + 8 * r);
  }
  const bool ok = pos >= 0 && pos < a.max_ctx;
  if (!ok && split == 0 && g == 0 && tid == 0) flag_error(a.err, QA_DEVERR_POSITION);

  // ---- 2. the cache tiles, two in flight ahead of the one being used.
  // Rows [0, pos) -- all before the new slot -- in ns near-equal runs; keys
  // past the run are clamped to its last row (read again, their scores
  // masked), so every wave issues a fixed number of loads.  K: tile t, lane l
  // holds dims 32 ks + 8 (l/16) .. +7 of key 16 t + kperm(l%16) (row l%16 of
  // the A operand of k-step ks).  V: lane (kg, c) holds dims 8c .. 8c+7 of
  // keys 16 t + kg + 4u, u < 4.
  const int nrows = ok ? pos : 0;
  const int k0 = (int)((long)split * nrows / ns);
  const int k1 = (int)((long)(split + 1) * nrows / ns);
  const int klast = max(k1 - 1, 0);
  const uint16_t* kbase = a.c.k + (size_t)b * a.c.sb + (size_t)g * a.c.sh;
  const uint16_t* vbase = a.c.v + (size_t)b * a.c.sb + (size_t)g * a.c.sh;
  // A-operand row m holds key (m >> 2) + 4 (m & 3): score register r of lane
  // (kb, n) is then key kb + 4 r, the key that lane's V rows hold
  const int kperm = (c >> 2) + 4 * (c & 3);
  u32x4 kq[TPW][4], vr[TPW][4];
  auto issue = [&](int i) {
    const int t0 = k0 + 16 * (w + NW * i);
    const uint16_t* kr = kbase + (size_t)min(t0 + kperm, klast) * a.c.sp + 8 * kg;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) kq[i][ks] = ld16(kr + 32 * ks);
#pragma unroll
    for (int u = 0; u < 4; ++u)
      vr[i][u] = ld16(vbase + (size_t)min(t0 + kg + 4 * u, klast) * a.c.sp + 8 * c);
  };
  // q' for every head into the wave's patch (its inputs arrive with the
  // position), ahead of the cache loads so that nothing after them waits
  qr.compute(a, pos, lane, sq);
  // the new token's k' (fp64, one RNE) into its slot, before this wave's
  // own cache loads
  float kn0 = 0.f, kn1 = 0.f;  // the new k' (bf16 values), elements lane, lane+64
  if (nt_wave && ok) {
    double sn, cn;
    sincos((double)pos * qr.invf, &sn, &cn);
    const double wk0 = a.k_norm_w ? (double)bf_to_f(nw0) : 1.0;
    const double wk1 = a.k_norm_w ? (double)bf_to_f(nw1) : 1.0;
    uint16_t o0, o1;
    kprime_pair(nk0, nk1, wk0, wk1, a.eps, cn, sn, &o0, &o1);
    const size_t crow = (size_t)b * a.c.sb + (size_t)g * a.c.sh + (size_t)pos * a.c.sp;
    a.c.k[crow + lane] = o0;
    a.c.k[crow + lane + 64] = o1;
    if (c == 0) {
#pragma unroll
      for (int r = 0; r < 4; ++r) st16(a.c.v + crow + 32 * kg + 8 * r, nv[r]);
    }
    kn0 = bf_to_f(o0);
    kn1 = bf_to_f(o1);
  }
  issue(0);
  if (TPW > 1) issue(1);

  // ---- 3. the new token's scores
  wave_lds_sync();  // the wave's q' patch
  float snew[G];
#pragma unroll
  for (int h = 0; h < G; ++h) snew[h] = ninf;
  if (nt_wave && ok) {
#pragma unroll
    for (int h = 0; h < G; ++h)
      snew[h] = row16_sum(bf_to_f(sq[h][lane]) * kn0 + bf_to_f(sq[h][lane + 64]) * kn1);
#pragma unroll
    for (int h = 0; h < G; ++h)
      snew[h] = (__int_as_float(__builtin_amdgcn_readlane(__float_as_int(snew[h]), 0)) +
                 __int_as_float(__builtin_amdgcn_readlane(__float_as_int(snew[h]), 16))) +
                (__int_as_float(__builtin_amdgcn_readlane(__float_as_int(snew[h]), 32)) +
                 __int_as_float(__builtin_amdgcn_readlane(__float_as_int(snew[h]), 48)));
  }
  u32x4 qv[4];  // the B operand: q' of head l%16, dims 32 ks + 8 (l/16) .. +7
  {
    const int qh = min(lane & 15, G - 1);
    const bool qvalid = (lane & 15) < G;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      qv[ks] = ld16(&sq[qh][32 * ks + 8 * (lane >> 4)]);
      if (!qvalid) qv[ks] = u32x4{0u, 0u, 0u, 0u};
    }
  }

  // ---- 4. the wave's tiles in arrival order, online softmax per head.
  // Lane (kb, n) = (l/16, l%16) holds head n's scores of keys kb + 4 r of the
  // tile (S^T register r), which are also the B operand (P^T) of the
  // 16x16x16 P.V product: its K index 4 kb + r is key kb + 4 r.  The A
  // operand (V^T) of output dims 8 m + j, j < 8, takes from lane (kb, m) the
  // bf16 j of its V rows kb + 4 r.  So lane (kb, n) accumulates dims
  // 32 kb + 8 r + j of head n in acc[j][r].  Its running max and sum are
  // head n's (equal in the four lanes of the head); lanes of heads n >= G see
  // a zero q' and are never stored.
  const int n_h = c;
  float mrun = ninf, lrun = 0.f;
  f32x4 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int t0 = k0 + 16 * (w + NW * i);
    if (t0 < k1) {  // (wave-uniform; key t0 is in the run)
      f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) sc = mfma16x16x32(kq[i][ks], qv[ks], sc);
      float tm = ninf;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        sc[r] = t0 + kg + 4 * r < k1 ? sc[r] : ninf;
        tm = fmaxf(tm, sc[r]);
      }
      const float mnew = fmaxf(mrun, rows4_max(tm));
      const float alpha = __builtin_amdgcn_exp2f(mrun - mnew);  // 0 while mrun = -inf
      float pr[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) pr[r] = __builtin_amdgcn_exp2f(sc[r] - mnew);
      lrun = lrun * alpha + rows4_add((pr[0] + pr[1]) + (pr[2] + pr[3]));
      mrun = mnew;
      if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {  // (wave-uniform)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] *= alpha;
      }
      const u32x2 pb = {pack_bf16x2(pr[0], pr[1]), pack_bf16x2(pr[2], pr[3])};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int e2 = j >> 1;
        const uint32_t v0 = vr[i][0][e2], v1 = vr[i][1][e2];
        const uint32_t v2 = vr[i][2][e2], v3 = vr[i][3][e2];
        // bf16 j of rows (u, u+1): bytes 0-1 (j even) or 2-3 (j odd) of each
        const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
        const u32x2 av = {__builtin_amdgcn_perm(v1, v0, sel), __builtin_amdgcn_perm(v3, v2, sel)};
        acc[j] = mfma16x16x16(av, pb, acc[j]);
      }
    }
    if (i + 2 < TPW) issue(i + 2);
  }
  // the new key: one more step of the online softmax (its weight in fp32),
  // its value added once
  if (nt_wave && ok) {
    float sn = snew[0];
#pragma unroll
    for (int h = 1; h < G; ++h) sn = n_h == h ? snew[h] : sn;
    const float mnew = fmaxf(mrun, sn);
    const float alpha = mrun == ninf ? 0.f : __builtin_amdgcn_exp2f(mrun - mnew);
    const float pn = __builtin_amdgcn_exp2f(sn - mnew);
    lrun = lrun * alpha + pn;
    mrun = mnew;
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t vw = nv[r][j >> 1];
        acc[j][r] = acc[j][r] * alpha + pn * ((j & 1) ? bf_hi(vw) : bf_lo(vw));
      }
  }
  // the wave's (max, sum, output) for the combine
  if (n_h < G) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float* d = &s_red[w][n_h][32 * kg + 8 * r];
      *reinterpret_cast<float4*>(d) = make_float4(acc[0][r], acc[1][r], acc[2][r], acc[3][r]);
      *reinterpret_cast<float4*>(d + 4) = make_float4(acc[4][r], acc[5][r], acc[6][r], acc[7][r]);
    }
    if (kg == 0) {
      s_m[w][n_h] = mrun;
      s_l[w][n_h] = lrun;
    }
  }
  __syncthreads();

  // ---- 5. the split's partial: the waves combined at their common max
  if (tid < G * 32) {
    const int hl = tid >> 5, d4 = (tid & 31) * 4;
    float m = ninf;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) m = fmaxf(m, s_m[ww][hl]);
    float l = 0.f;
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
    if (m != ninf) {
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) {
        const float mw = s_m[ww][hl];
        const float wgt = mw == ninf ? 0.f : __builtin_amdgcn_exp2f(mw - m);
        const float4 t = *reinterpret_cast<const float4*>(&s_red[ww][hl][d4]);
        l += wgt * s_l[ww][hl];
        o.x += wgt * t.x; o.y += wgt * t.y; o.z += wgt * t.z; o.w += wgt * t.w;
      }
    }
    *reinterpret_cast<float4*>(a.part_o + (rowbase + hl) * kHeadDim + d4) = o;
    if ((tid & 31) == 0) {
      a.part_m[rowbase + hl] = m;
      a.part_l[rowbase + hl] = l;
    }
  }
  if constexpr (SYNC) merge_pair<64 * kDecodeWaves, 1>(a, pair, b, g, G);
}

template <int G, int TPW>
static void launch_tpw(const DecodeArgs& a, const RopeFreq& f, hipStream_t s) {
  const dim3 grid(a.n_split * a.n_kv_heads * a.batch);
  if (a.sync)
    hipLaunchKernelGGL((decode_kernel<G, TPW, true>), grid, dim3(64 * kDecodeWaves), 0, s, a, f);
  else
    hipLaunchKernelGGL((decode_kernel<G, TPW, false>), grid, dim3(64 * kDecodeWaves), 0, s, a, f);
}

template <int G>
static hipError_t launch_decode_g(const DecodeArgs& a, const RopeFreq& f, hipStream_t s) {
  const int nt = a.keys_per_split / 16;
  if (a.keys_per_split % 16 != 0 || nt < 1 || nt > kDecodeMaxTiles || a.n_split < 1 ||
      (long)a.n_split * a.keys_per_split < a.max_ctx - 1)
    return hipErrorInvalidValue;
  switch ((nt + kDecodeWaves - 1) / kDecodeWaves) {
    case 1: launch_tpw<G, 1>(a, f, s); break;
    case 2: launch_tpw<G, 2>(a, f, s); break;
    case 3: launch_tpw<G, 3>(a, f, s); break;
    case 4: launch_tpw<G, 4>(a, f, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, const RopeFreq& f, int group,
                         hipStream_t s, int* n_kernels) {
  *n_kernels = 0;
  if (a.sync && ((a.batch * a.n_kv_heads) % 8 != 0 || a.n_split > kInlineMaxSplits))
    return hipErrorInvalidValue;  // the grid numbering and the counter fields
  hipError_t e;
  switch (group) {
    case 1: e = launch_decode_g<1>(a, f, s); break;
    case 2: e = launch_decode_g<2>(a, f, s); break;
    case 4: e = launch_decode_g<4>(a, f, s); break;
    case 8: e = launch_decode_g<8>(a, f, s); break;
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
