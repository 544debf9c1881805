// Hidden-state RMSNorm with the residual add, in the reference's cast
// placement.
//
// "dryft-flash-infer" agent guide, Where the wins are (RMSNorm, small and
// repeated, safe to fuse) and Numerics (reductions may be reordered; where the
// bf16 cast happens may not move).  The reference model's norm casts the
// normalised value to bf16 before it multiplies by the bf16 weight, and its
// residual stream is a bf16 tensor, so:
//   r   = bf16(x + residual)                 (r = x without a residual)
//   out = bf16(w * bf16(r / sqrt(mean(r^2) + eps)))
// with every other step exact.  Each rounding to bf16 is one round to
// nearest even of the exact value:
// - the sum of two bf16 values is formed in fp32: it is exact there unless
//   the smaller term is below 2^-15 of the larger, and then too small to
//   move the bf16 rounding, so rounding the fp32 sum once gives the bf16 of
//   the exact sum; the product of two bf16 values (16 significant bits) is
//   exact in fp32 in the normal range;
// - the sum of squares is accumulated in fp64 (reordered: it differs from
//   another order by ~1e-16 relative);
// - r / s is formed in fp32 as r * (1/s) and rounded from there unless it
//   lies within 8 fp32 ulps of a bf16 rounding midpoint (its error is at
//   most ~3 2^-24 relative, under 2 ulps), where the correctly rounded fp64
//   division decides; values that are not finite or near the subnormal range
//   take the fp64 steps too.
//
// One wave per token row: all loads of the row first (CH 16-byte pieces per
// lane, CH = ceil(hidden / 512), a template argument so that registers are
// sized for the row at hand), the sum of squares reduced across the wave,
// then the row written back.  Batches of at most kNormRowTokens rows spread
// each row over a workgroup instead (rmsnorm_row_kernel).  The traffic is 2
// bytes per element for each of x, residual in, out and residual out.
#include <utility>

#include "qa.h"
#include "qa_device.h"
#include "rmsnorm.h"

namespace qa {

// fp64 -> bf16 bits, one round to nearest even: for |x| >= 2^-126 (finite)
// on the integer bits (8 significant bits kept, a carry may step the
// exponent; the result converts to fp32 exactly or overflows to inf), else
// through the general routine (zero, subnormal, inf, NaN).
__device__ __forceinline__ uint16_t rne_bf16(double x) {
  const uint64_t u = (uint64_t)__double_as_longlong(x);
  const uint32_t be = (uint32_t)(u >> 52) & 0x7FFu;
  if (be >= 897u && be < 0x7FFu) {
    const uint64_t r =
        (u + 0x00000FFFFFFFFFFFull + ((u >> 45) & 1u)) & ~0x00001FFFFFFFFFFFull;
    return (uint16_t)(__float_as_uint((float)__longlong_as_double((long long)r)) >> 16);
  }
  return f64_to_bf16_rne(x);
}

// fp32 -> bf16 bits, round to nearest even, for a finite or infinite value.
__device__ __forceinline__ uint16_t rne16(float f) {
  const uint32_t u = __float_as_uint(f);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// Whether the fp32 value f leaves the fast path: not finite, or below 2^-118
// in magnitude (near the subnormal range, where fp32 products lose bits).
__device__ __forceinline__ bool off_range(float f) {
  const uint32_t e = (__float_as_uint(f) >> 23) & 0xFFu;
  return e < 9u || e == 0xFFu;
}

__device__ __forceinline__ uint16_t half_of(const u32x4& v, int e) {
  const uint32_t w = v[e >> 1];
  return (uint16_t)((e & 1) ? (w >> 16) : (w & 0xffffu));
}

// The 8 values of one 16-byte piece: r = bf16(x + residual) (r = x without
// a residual), formed in fp32 (exact for a finite sum; an overflowing sum or
// a NaN takes the fp64 steps), their squares added to ss in fp64.
__device__ __forceinline__ u32x4 add_piece(u32x4 x, u32x4 res, bool has_res, double& ss) {
  u32x4 out;
#pragma unroll
  for (int e2 = 0; e2 < 4; ++e2) {
    uint16_t r[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint16_t xb = half_of(x, 2 * e2 + h);
      r[h] = xb;
      if (has_res) {
        const float xf = bf_to_f(xb), rf = bf_to_f(half_of(res, 2 * e2 + h));
        const float sf = xf + rf;
        r[h] = ((__float_as_uint(sf) >> 23) & 0xFFu) == 0xFFu ? rne_bf16((double)xf + (double)rf)
                                                              : rne16(sf);
      }
      const double rv = (double)bf_to_f(r[h]);
      ss += rv * rv;
    }
    out[e2] = (uint32_t)r[0] | ((uint32_t)r[1] << 16);
  }
  return out;
}

// out = bf16(w * bf16(r / s)) (no weight: bf16(r / s)) for the 8 values of a
// piece, inv = 1/s rounded to fp32.  r / s is formed as r * inv and rounded
// from there unless it lies within 8 fp32 ulps of a bf16 rounding midpoint
// (its error is under 2 ulps) or outside the fast range, where the correctly
// rounded fp64 division decides; w * bf16(r / s) is exact in fp32 in range.
__device__ __forceinline__ u32x4 norm_piece(u32x4 r, u32x4 w, bool has_w, double s,
                                            float inv) {
  u32x4 o;
#pragma unroll
  for (int e2 = 0; e2 < 4; ++e2) {
    uint16_t ob[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int e = 2 * e2 + h;
      const float rv = bf_to_f(half_of(r, e));
      const float q = rv * inv;
      const uint32_t lo = __float_as_uint(q) & 0xFFFFu;
      // (a zero quotient is exact, or rounds to zero in fp64 too)
      const bool exact_div =
          (off_range(q) && q != 0.f) || (lo > 0x8000u - 8u && lo < 0x8000u + 8u);
      const uint16_t yb = exact_div ? rne_bf16((double)rv / s) : rne16(q);
      ob[h] = yb;
      if (has_w) {
        const float wf = bf_to_f(half_of(w, e));
        const float p = wf * bf_to_f(yb);
        ob[h] = off_range(p) && p != 0.f ? rne_bf16((double)wf * (double)bf_to_f(yb))
                                         : rne16(p);
      }
    }
    o[e2] = (uint32_t)ob[0] | ((uint32_t)ob[1] << 16);
  }
  return o;
}

// The weights load after the residual add, once x and the residual are
// dead; rows of up to 5 pieces per lane (hidden <= 2560) then fit six waves
// per SIMD without spilling.
template <int CH>
__global__ __launch_bounds__(256, CH <= 5 ? 6 : 1) void rmsnorm_hidden_kernel(NormArgs a) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= a.n_tokens) return;  // (wave-uniform)
  const int nc = a.hidden >> 3;  // 16-byte pieces in a row
  const size_t row = (size_t)t * a.hidden;
  u32x4 xr[CH], rr[CH], wr[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int i = lane + 64 * c;
    if (i < nc) {
      xr[c] = ld16(a.x + row + 8 * i);
      if (a.res) rr[c] = ld16(a.res + row + 8 * i);
    }
  }
  double ss = 0.0;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int i = lane + 64 * c;
    if (i < nc) rr[c] = add_piece(xr[c], rr[c], a.res != nullptr, ss);
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int i = lane + 64 * c;
    if (i < nc && a.w) wr[c] = ld16(a.w + 8 * i);
  }
  ss = wave_sum(ss);
  const double s = sqrt(ss / (double)a.hidden + a.eps);
  const float inv = (float)(1.0 / s);
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int i = lane + 64 * c;
    if (i < nc) {
      st16(a.out + row + 8 * i, norm_piece(rr[c], wr[c], a.w != nullptr, s, inv));
      if (a.res) st16(a.res + row + 8 * i, rr[c]);
    }
  }
}

// Up to kNormRowTokens rows: one workgroup per row and one 16-byte piece per
// thread, so a row's serial work is one piece deep instead of hidden/512
// pieces; the waves' sums of squares meet in LDS and are added in wave order.
__global__ __launch_bounds__(1024) void rmsnorm_row_kernel(NormArgs a) {
  __shared__ double s_ss[16];
  const int i = threadIdx.x, w = i >> 6, nw = blockDim.x >> 6;
  const int nc = a.hidden >> 3;
  const size_t row = (size_t)blockIdx.x * a.hidden;
  const bool on = i < nc;
  u32x4 xr = {0u, 0u, 0u, 0u}, rr = xr, wr = xr;
  if (on) {
    xr = ld16(a.x + row + 8 * i);
    if (a.res) rr = ld16(a.res + row + 8 * i);
    if (a.w) wr = ld16(a.w + 8 * i);
  }
  double ss = 0.0;
  if (on) rr = add_piece(xr, rr, a.res != nullptr, ss);
  ss = wave_sum(ss);
  if ((i & 63) == 0) s_ss[w] = ss;
  __syncthreads();
  double tot = 0.0;
  for (int v = 0; v < nw; ++v) tot += s_ss[v];
  const double s = sqrt(tot / (double)a.hidden + a.eps);
  if (on) {
    st16(a.out + row + 8 * i, norm_piece(rr, wr, a.w != nullptr, s, (float)(1.0 / s)));
    if (a.res) st16(a.res + row + 8 * i, rr);
  }
}

template <int CH>
static void launch_one(const NormArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((rmsnorm_hidden_kernel<CH>), dim3((a.n_tokens + 3) / 4), dim3(256), 0, s,
                     a);
}

template <int... CH>
static hipError_t launch_ch(const NormArgs& a, hipStream_t s,
                            std::integer_sequence<int, CH...>) {
  const int ch = (a.hidden + 511) / 512;
  if (ch < 1 || ch > kNormMaxChunks) return hipErrorInvalidValue;
  ((ch == CH + 1 ? launch_one<CH + 1>(a, s) : void()), ...);
  return hipGetLastError();
}

hipError_t launch_rmsnorm_hidden(const NormArgs& a, hipStream_t s) {
  if (a.n_tokens == 0) return hipSuccess;
  if (a.n_tokens <= kNormRowTokens) {
    const int nc = a.hidden >> 3;
    if (nc < 1 || nc > 1024) return hipErrorInvalidValue;
    hipLaunchKernelGGL(rmsnorm_row_kernel, dim3(a.n_tokens), dim3(64 * ((nc + 63) / 64)), 0, s,
                       a);
    return hipGetLastError();
  }
  return launch_ch(a, s, std::make_integer_sequence<int, kNormMaxChunks>{});
}

}  // namespace qa
