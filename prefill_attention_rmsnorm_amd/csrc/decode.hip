// Single-token decode on gfx950: split-K over the cache, memory-bound.
//
// "dryft-flash-infer" agent guide, Where the wins are: per-step overhead and
// the preallocated, strided cache.  Every workgroup owns (split, kv head,
// sequence).  It first issues all of its cache loads with 16-byte loads,
// then, while they are in flight, forms q' for the G query heads of the
// group; the workgroup whose split holds the new slot also runs the K
// prologue for it (fp64, one RNE), writes the slot to the cache and scores it
// from LDS.  Scores are a 16x16x32 bf16 MFMA (heads x keys, K loaded straight
// into the B-operand layout); the softmax weights of key pairs are packed as
// bf16x2 so P.V runs on dot2 instructions over the V rows as loaded.  The
// workgroup writes a partial (max, sum, unnormalised output) that merge.hip
// combines.
#include "qa.h"
#include "qa_device.h"

namespace qa {

template <int G, int KS>
__global__ __launch_bounds__(256) void decode_kernel(DecodeArgs a, RopeFreq f) {
  constexpr int NWM = KS / 32;  // waves that form scores (32 keys each)
  constexpr int NV = KS / 16;   // V rows per thread (16 key groups x NV = KS)
  static_assert(KS == 64 || KS == 128, "split length");
  static_assert(G <= 8, "group");
  __shared__ __attribute__((aligned(16))) uint16_t s_q[G][kHeadDim];
  __shared__ float s_knew[kHeadDim];
  __shared__ float s_vnew[kHeadDim];
  __shared__ float s_snew[G];
  __shared__ float s_max[NWM][8];
  __shared__ float s_sum[NWM][8];
  __shared__ __attribute__((aligned(16))) uint32_t s_pp[NWM][16][8];
  __shared__ __attribute__((aligned(16))) float s_acc[16][16][G][8];

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int pos = a.positions[b];
  const bool ok = pos >= 0 && pos < a.max_ctx;
  if (!ok && split == 0 && g == 0 && tid == 0)
    flag_error(a.err, QA_DEVERR_POSITION);
  const int ctx = ok ? pos + 1 : 0;
  const int k0 = split * KS, k1 = min(k0 + KS, ctx);
  const size_t pairidx = (size_t)b * a.n_kv_heads + g;
  const size_t rowbase = (pairidx * a.n_split + split) * G;
  const float ninf = -__builtin_inff();

  if (k0 >= k1) {  // nothing to attend in this split
    if (tid < G) {
      a.part_m[rowbase + tid] = ninf;
      a.part_l[rowbase + tid] = 0.f;
    }
    return;
  }
  // The new slot (pos) is not read from the cache: it is written by this
  // call.  The workgroup that owns it scores it from LDS instead.
  const bool owner = pos >= k0 && pos < k1;
  const int kload = owner ? pos : k1;  // cache rows [k0, kload) are read
  const bool any_load = kload > k0;
  const uint16_t* kbase = a.c.k + (size_t)b * a.c.sb + (size_t)g * a.c.sh;
  const uint16_t* vbase = a.c.v + (size_t)b * a.c.sb + (size_t)g * a.c.sh;

  // ---- 1. loads.  The prologue's inputs are loaded first: the memory
  // counter is waited on in issue order, so anything loaded after the cache
  // rows could only be used once the whole cache read had landed.
  const double invf = f.inv_freq[lane];  // (a lane-indexed kernel-argument load)
  constexpr int HPW = (G + 3) / 4;  // query heads per wave
  uint16_t qx0[HPW], qx1[HPW];
#pragma unroll
  for (int i = 0; i < HPW; ++i) {
    const int hl = min(w + 4 * i, G - 1);
    const uint16_t* qr = a.q + ((size_t)b * a.n_q_heads + g * G + hl) * kHeadDim;
    qx0[i] = qr[lane];
    qx1[i] = qr[lane + 64];
  }
  // norm weights and the new token's k/v are loaded unconditionally from
  // valid addresses (the values are selected afterwards), so no branch sits
  // between the loads
  const uint16_t* qwp = a.q_norm_w ? a.q_norm_w : a.q;
  const uint16_t* kwp = a.k_norm_w ? a.k_norm_w : a.q;
  const uint16_t qw0r = qwp[lane], qw1r = qwp[lane + 64];
  const uint16_t kw0r = kwp[lane], kw1r = kwp[lane + 64];
  const uint16_t* kr0 = a.k + pairidx * kHeadDim;
  const uint16_t kx0 = kr0[lane], kx1 = kr0[lane + 64];
  const uint32_t vx = reinterpret_cast<const uint32_t*>(a.v + pairidx * kHeadDim)[lane];
  __builtin_amdgcn_sched_barrier(0);  // the small loads stay first
  // Cache rows past kload are clamped to kload-1 (a written slot whose score
  // is masked); when the split holds only the new slot the clamped row 0 is
  // read but never used.
  const int klast = max(kload - 1, 0);
  // K, for the score waves, in the B-operand layout of the 16x16x32 MFMA:
  // lane l holds dims 32*ks + 8*(l/16) .. +7 of key 16*j + l%16.
  u32x4 kq[2][4];
  {
    const int wk = min(w, NWM - 1);  // waves past NWM load (and drop) a copy
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int key = min(k0 + 32 * wk + 16 * j + (lane & 15), klast);
      const uint16_t* kr = kbase + (size_t)key * a.c.sp + 8 * (lane >> 4);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) kq[j][ks] = ld16(kr + 32 * ks);
    }
  }
  // V, for every thread: 8 dims (chunk c) of keys kg + 16*i.
  const int kg = tid >> 4, c = tid & 15;
  u32x4 vr[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int key = min(k0 + kg + 16 * i, klast);
    vr[i] = ld16(vbase + (size_t)key * a.c.sp + 8 * c);
  }
  // keep the loads in this order, ahead of the prologue arithmetic
  __builtin_amdgcn_sched_barrier(0);

  // ---- 2. prologue while the cache loads are in flight
  {
    const double ang = (double)pos * invf;
    float s32, c32;
    sincos_reduced(ang, &s32, &c32);
    const float w0 = a.q_norm_w ? bf_to_f(qw0r) : 1.f;
    const float w1 = a.q_norm_w ? bf_to_f(qw1r) : 1.f;
#pragma unroll
    for (int i = 0; i < HPW; ++i) {
      const int hl = w + 4 * i;
      if (hl >= G) break;
      const float x0 = bf_to_f(qx0[i]), x1 = bf_to_f(qx1[i]);
      const float ss = wave_sum(x0 * x0 + x1 * x1);
      const float rinv = 1.0f / sqrtf(ss * (1.0f / 128.0f) + (float)a.eps);
      const float y0 = x0 * rinv * w0, y1 = x1 * rinv * w1;
      const uint32_t pk = pack_bf16x2((y0 * c32 - y1 * s32) * a.qscale,
                                      (y1 * c32 + y0 * s32) * a.qscale);
      s_q[hl][lane] = (uint16_t)(pk & 0xffffu);
      s_q[hl][lane + 64] = (uint16_t)(pk >> 16);
    }
    if (owner && w == 0) {
      double sn, cn;
      sincos(ang, &sn, &cn);
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
      s_vnew[2 * lane] = bf_lo(vx);
      s_vnew[2 * lane + 1] = bf_hi(vx);
    }
  }
  __syncthreads();

  // ---- 3. scores.  Waves w < NWM: S = q' K^T for keys k0 + 32w + [0, 32)
  // with the heads on the MFMA row axis: lane l holds head 4*(l/16) + r of
  // key l%16 (+16 for the second tile).
  const int hrow = 4 * (lane >> 4);  // first head of this lane's registers
  f32x4 sj[2];
  if (w < NWM) {
    const int qh = min(lane & 15, G - 1);
    const bool qvalid = (lane & 15) < G;
    sj[0] = f32x4{0.f, 0.f, 0.f, 0.f};
    sj[1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      u32x4 qa = ld16(&s_q[qh][32 * ks + 8 * (lane >> 4)]);
      if (!qvalid) qa = u32x4{0u, 0u, 0u, 0u};
      sj[0] = mfma16x16x32(qa, kq[0][ks], sj[0]);
      sj[1] = mfma16x16x32(qa, kq[1][ks], sj[1]);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const bool kok = k0 + 32 * w + 16 * j + (lane & 15) < kload;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (!kok || hrow + r >= G) sj[j][r] = ninf;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float mx = row16_max(fmaxf(sj[0][r], sj[1][r]));
      if ((lane & 15) == 0 && hrow + r < G) s_max[w][hrow + r] = mx;
    }
  }
  if (owner) {  // scores of the new slot, one wave per head
    for (int hl = w; hl < G; hl += 4) {
      float d = bf_to_f(s_q[hl][lane]) * s_knew[lane] +
                bf_to_f(s_q[hl][lane + 64]) * s_knew[lane + 64];
      d = wave_sum(d);
      if (lane == 0) s_snew[hl] = d;
    }
  }
  __syncthreads();

  // ---- 4. softmax weights: p = exp2(s - M) with M the split's max per head.
  // Pairs (key, key+16) are packed as bf16x2 for the P.V dot products.
  if (w < NWM) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = min(hrow + r, G - 1);
      float mh = s_max[0][h];
#pragma unroll
      for (int ww = 1; ww < NWM; ++ww) mh = fmaxf(mh, s_max[ww][h]);
      if (owner) mh = fmaxf(mh, s_snew[h]);
      const float p0 = __builtin_amdgcn_exp2f(sj[0][r] - mh);
      const float p1 = __builtin_amdgcn_exp2f(sj[1][r] - mh);
      const float sum = row16_sum(p0 + p1);
      if (hrow + r < G) {
        s_pp[w][lane & 15][hrow + r] = pack_bf16x2(p0, p1);
        if ((lane & 15) == 0) s_sum[w][hrow + r] = sum;
      }
    }
  }
  __syncthreads();

  // ---- 5. O += P.V: thread (kg, c) over its key pairs (kg + 32m, kg + 32m + 16)
  float acc[G][8];
#pragma unroll
  for (int hl = 0; hl < G; ++hl)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[hl][e] = 0.f;
  if (any_load) {  // (uniform) with only the new slot there is nothing to add
#pragma unroll
  for (int m = 0; m < NWM; ++m) {
    uint32_t pp[G];
#pragma unroll
    for (int hl = 0; hl < G; ++hl) pp[hl] = s_pp[m][kg][hl];
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) {
      const uint32_t va = vr[2 * m][e2], vb2 = vr[2 * m + 1][e2];
      const uint32_t lo = (va & 0xffffu) | (vb2 << 16);
      const uint32_t hi = (va >> 16) | (vb2 & 0xffff0000u);
#pragma unroll
      for (int hl = 0; hl < G; ++hl) {
        acc[hl][2 * e2] = dot2_bf16(pp[hl], lo, acc[hl][2 * e2]);
        acc[hl][2 * e2 + 1] = dot2_bf16(pp[hl], hi, acc[hl][2 * e2 + 1]);
      }
    }
  }
  }
#pragma unroll
  for (int hl = 0; hl < G; ++hl)
#pragma unroll
    for (int e4 = 0; e4 < 2; ++e4)
      *reinterpret_cast<float4*>(&s_acc[kg][c][hl][4 * e4]) =
          make_float4(acc[hl][4 * e4], acc[hl][4 * e4 + 1], acc[hl][4 * e4 + 2],
                      acc[hl][4 * e4 + 3]);
  __syncthreads();

  // ---- 6. the split's partial (the new slot, if owned, added here)
  if (tid < G * 32) {
    const int hl = tid >> 5, d4 = (tid & 31) * 4;
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const float4 t = *reinterpret_cast<const float4*>(
          &s_acc[q][d4 >> 3][hl][d4 & 7]);
      o.x += t.x; o.y += t.y; o.z += t.z; o.w += t.w;
    }
    float mh = s_max[0][hl], L = s_sum[0][hl];
#pragma unroll
    for (int ww = 1; ww < NWM; ++ww) {
      mh = fmaxf(mh, s_max[ww][hl]);
      L += s_sum[ww][hl];
    }
    if (owner) {
      mh = fmaxf(mh, s_snew[hl]);
      const float pn = __builtin_amdgcn_exp2f(s_snew[hl] - mh);
      L += pn;
      o.x += pn * s_vnew[d4]; o.y += pn * s_vnew[d4 + 1];
      o.z += pn * s_vnew[d4 + 2]; o.w += pn * s_vnew[d4 + 3];
    }
    *reinterpret_cast<float4*>(a.part_o + (rowbase + hl) * kHeadDim + d4) = o;
    if ((tid & 31) == 0) {
      a.part_m[rowbase + hl] = mh;
      a.part_l[rowbase + hl] = L;
    }
  }
}

template <int G>
static hipError_t launch_decode_g(const DecodeArgs& a, const RopeFreq& f,
                                  hipStream_t s) {
  const dim3 grid(a.n_split, a.n_kv_heads, a.batch);
  if (a.keys_per_split == 64)
    hipLaunchKernelGGL((decode_kernel<G, 64>), grid, dim3(256), 0, s, a, f);
  else if (a.keys_per_split == 128)
    hipLaunchKernelGGL((decode_kernel<G, 128>), grid, dim3(256), 0, s, a, f);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, const RopeFreq& f, int group,
                         hipStream_t s, int* n_kernels) {
  *n_kernels = 0;
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
  e = launch_merge(a, group, s);
  if (e == hipSuccess) *n_kernels = 2;
  return e;
}

}  // namespace qa
