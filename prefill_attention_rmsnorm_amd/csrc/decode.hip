// Single-token decode on gfx950: split-K over the cache, memory-bound.
//
// "dryft-flash-infer" agent guide, Where the wins are: per-step overhead and
// the preallocated, strided cache.  One launch per call: every workgroup owns
// (split, kv head, sequence), streams its keys with 16-byte loads (16 lanes
// cover one 256-byte K or V row), forms the G query heads' scores with bf16
// dot2 instructions and row reductions over DPP, and writes a partial
// (max, sum, unnormalised output).  The workgroup owning the new slot also
// runs the prologue for it (k' in fp64, one RNE) and writes the cache.  The
// last workgroup of a (sequence, kv head) to finish merges the partials by
// log-sum-exp in split order, so results do not depend on arrival order.
#include "qa.h"
#include "qa_device.h"

namespace qa {

template <int G, int KS>
__global__ __launch_bounds__(256) void decode_kernel(DecodeArgs a, RopeFreq f) {
  constexpr int KPT = KS / 16;  // keys per thread
  __shared__ __attribute__((aligned(16))) uint16_t s_q[G][kHeadDim];
  __shared__ __attribute__((aligned(16))) uint16_t s_knew[kHeadDim];
  __shared__ __attribute__((aligned(16))) uint16_t s_vnew[kHeadDim];
  __shared__ float s_red[4][G];
  __shared__ float s_acc[4][16][G][8];
  __shared__ int s_last;

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int pos = a.positions[b];
  const bool ok = pos >= 0 && pos < a.max_ctx;
  if (!ok && split == 0 && g == 0 && tid == 0)
    flag_error(a.err, QA_DEVERR_POSITION);
  const int ctx = ok ? pos + 1 : 0;
  const int k0 = split * KS, k1 = min(k0 + KS, ctx);
  const bool owner = ok && (pos / KS == split);
  const size_t pairidx = (size_t)b * a.n_kv_heads + g;
  const size_t rowbase = (pairidx * a.n_split + split) * G;

  if (k0 < k1) {
    // ---- prologue: q' for the G heads of the group, k'/v of the new slot
    {
      double sn, cn;
      sincos((double)pos * f.inv_freq[lane], &sn, &cn);
      const float c32 = (float)cn, s32 = (float)sn;
      const float w0 = a.q_norm_w ? bf_to_f(a.q_norm_w[lane]) : 1.f;
      const float w1 = a.q_norm_w ? bf_to_f(a.q_norm_w[lane + 64]) : 1.f;
      for (int hl = w; hl < G; hl += 4) {
        const uint16_t* qr = a.q + ((size_t)b * a.n_q_heads + g * G + hl) * kHeadDim;
        const float x0 = bf_to_f(qr[lane]), x1 = bf_to_f(qr[lane + 64]);
        const float ss = wave_sum(x0 * x0 + x1 * x1);
        const float rinv = 1.0f / sqrtf(ss * (1.0f / 128.0f) + (float)a.eps);
        const float y0 = x0 * rinv * w0, y1 = x1 * rinv * w1;
        const uint32_t pk = pack_bf16x2((y0 * c32 - y1 * s32) * a.qscale,
                                        (y1 * c32 + y0 * s32) * a.qscale);
        s_q[hl][lane] = (uint16_t)(pk & 0xffffu);
        s_q[hl][lane + 64] = (uint16_t)(pk >> 16);
      }
      if (owner && w == 0) {
        const uint16_t* kr = a.k + pairidx * kHeadDim;
        const double wk0 = a.k_norm_w ? (double)bf_to_f(a.k_norm_w[lane]) : 1.0;
        const double wk1 = a.k_norm_w ? (double)bf_to_f(a.k_norm_w[lane + 64]) : 1.0;
        uint16_t o0, o1;
        kprime_pair(kr[lane], kr[lane + 64], wk0, wk1, a.eps, cn, sn, &o0, &o1);
        s_knew[lane] = o0;
        s_knew[lane + 64] = o1;
        const size_t crow = (size_t)b * a.c.sb + (size_t)g * a.c.sh + (size_t)pos * a.c.sp;
        a.c.k[crow + lane] = o0;
        a.c.k[crow + lane + 64] = o1;
        const uint32_t vv = reinterpret_cast<const uint32_t*>(a.v + pairidx * kHeadDim)[lane];
        reinterpret_cast<uint32_t*>(s_vnew)[lane] = vv;
        reinterpret_cast<uint32_t*>(a.c.v + crow)[lane] = vv;
      }
    }
    __syncthreads();

    // ---- stream this split's keys: thread = (key group kg, 8-dim chunk c)
    const int kg = tid >> 4, c = tid & 15;
    const uint16_t* kb = a.c.k + (size_t)b * a.c.sb + (size_t)g * a.c.sh + 8 * c;
    const uint16_t* vb = a.c.v + (size_t)b * a.c.sb + (size_t)g * a.c.sh + 8 * c;
    u32x4 kr[KPT], vr[KPT];
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int key = k0 + kg + 16 * i;
      u32x4 xk = {0u, 0u, 0u, 0u}, xv = {0u, 0u, 0u, 0u};
      if (key < k1) {
        if (owner && key == pos) {
          xk = ld16(s_knew + 8 * c);
          xv = ld16(s_vnew + 8 * c);
        } else {
          xk = ld16(kb + (size_t)key * a.c.sp);
          xv = ld16(vb + (size_t)key * a.c.sp);
        }
      }
      kr[i] = xk;
      vr[i] = xv;
    }
    u32x4 qv[G];
#pragma unroll
    for (int hl = 0; hl < G; ++hl) qv[hl] = ld16(&s_q[hl][8 * c]);

    // ---- scores (log2 domain: scale*log2e is folded into q')
    const float ninf = -__builtin_inff();
    float sc[KPT][G];
    float mloc[G];
#pragma unroll
    for (int hl = 0; hl < G; ++hl) mloc[hl] = ninf;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const bool kok = k0 + kg + 16 * i < k1;
#pragma unroll
      for (int hl = 0; hl < G; ++hl) {
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t qe = qv[hl][e], ke = kr[i][e];
          d = dot2_bf16(qe, ke, d);
        }
        d = row16_sum(d);
        sc[i][hl] = kok ? d : ninf;
        mloc[hl] = fmaxf(mloc[hl], sc[i][hl]);
      }
    }
    float M[G];
#pragma unroll
    for (int hl = 0; hl < G; ++hl) {
      float mm = fmaxf(mloc[hl], __shfl_xor(mloc[hl], 16));
      mm = fmaxf(mm, __shfl_xor(mm, 32));
      if (lane == 0) s_red[w][hl] = mm;
    }
    __syncthreads();
#pragma unroll
    for (int hl = 0; hl < G; ++hl)
      M[hl] = fmaxf(fmaxf(s_red[0][hl], s_red[1][hl]), fmaxf(s_red[2][hl], s_red[3][hl]));
    __syncthreads();

    // ---- p = exp2(s - M), sum and P.V over this thread's keys and dims
    float acc[G][8], ls[G];
#pragma unroll
    for (int hl = 0; hl < G; ++hl) {
      ls[hl] = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[hl][e] = 0.f;
    }
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      float vf[8];
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        vf[2 * e2] = bf_lo(vr[i][e2]);
        vf[2 * e2 + 1] = bf_hi(vr[i][e2]);
      }
#pragma unroll
      for (int hl = 0; hl < G; ++hl) {
        const float pr = __builtin_amdgcn_exp2f(sc[i][hl] - M[hl]);
        ls[hl] += pr;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[hl][e] += pr * vf[e];
      }
    }
    // reduce over the 4 key groups of the wave (lanes with the same c)
#pragma unroll
    for (int hl = 0; hl < G; ++hl) {
      ls[hl] += __shfl_xor(ls[hl], 16);
      ls[hl] += __shfl_xor(ls[hl], 32);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        acc[hl][e] += __shfl_xor(acc[hl][e], 16);
        acc[hl][e] += __shfl_xor(acc[hl][e], 32);
      }
    }
    if (lane < 16) {
#pragma unroll
      for (int hl = 0; hl < G; ++hl)
#pragma unroll
        for (int e = 0; e < 8; ++e) s_acc[w][lane][hl][e] = acc[hl][e];
    }
    if (lane == 0) {
#pragma unroll
      for (int hl = 0; hl < G; ++hl) s_red[w][hl] = ls[hl];
    }
    __syncthreads();
    for (int idx = tid; idx < G * kHeadDim; idx += 256) {
      const int hl = idx >> 7, d = idx & 127;
      const float o = s_acc[0][d >> 3][hl][d & 7] + s_acc[1][d >> 3][hl][d & 7] +
                      s_acc[2][d >> 3][hl][d & 7] + s_acc[3][d >> 3][hl][d & 7];
      a.part_o[(rowbase + hl) * kHeadDim + d] = o;
    }
    if (tid == 0) {
#pragma unroll
      for (int hl = 0; hl < G; ++hl) {
        a.part_m[rowbase + hl] = M[hl];
        a.part_l[rowbase + hl] = s_red[0][hl] + s_red[1][hl] + s_red[2][hl] + s_red[3][hl];
      }
    }
  } else {
    if (tid < G) {
      a.part_m[rowbase + tid] = -__builtin_inff();
      a.part_l[rowbase + tid] = 0.f;
    }
  }

  // ---- the last workgroup of this (sequence, kv head) merges the splits
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const int prev = __hip_atomic_fetch_add(a.counters + pairidx, 1, __ATOMIC_ACQ_REL,
                                            __HIP_MEMORY_SCOPE_AGENT);
    s_last = (prev == a.n_split - 1);
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();

  const size_t pbase = pairidx * a.n_split * G;
  for (int idx = tid; idx < G * kHeadDim; idx += 256) {
    const int hl = idx >> 7, d = idx & 127;
    float Mx = -__builtin_inff();
    for (int s = 0; s < a.n_split; ++s) Mx = fmaxf(Mx, a.part_m[pbase + s * G + hl]);
    float L = 0.f, O = 0.f;
    if (Mx != -__builtin_inff()) {
      for (int s = 0; s < a.n_split; ++s) {
        const float ms = a.part_m[pbase + s * G + hl];
        if (ms == -__builtin_inff()) continue;
        const float wgt = __builtin_amdgcn_exp2f(ms - Mx);
        L += wgt * a.part_l[pbase + s * G + hl];
        O += wgt * a.part_o[(pbase + s * G + hl) * kHeadDim + d];
      }
    }
    const bool good = ok && L > 0.f;
    const float val = good ? O / L : 0.f;
    const size_t orow = ((size_t)b * a.n_q_heads + g * G + hl) * kHeadDim;
    reinterpret_cast<__bf16*>(a.out)[orow + d] = (__bf16)val;
    if (a.lse && d == 0)
      a.lse[(size_t)b * a.n_q_heads + g * G + hl] = good ? (Mx + __log2f(L)) * kLn2 : 0.f;
  }
  if (tid == 0)
    __hip_atomic_store(a.counters + pairidx, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
  if (e == hipSuccess) *n_kernels = 1;
  return e;
}

}  // namespace qa
