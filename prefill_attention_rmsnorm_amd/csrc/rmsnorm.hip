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
// with every other step exact.  The kernel computes in fp64: a sum of two
// bf16 values is exact there, and so is the product of two bf16 values; the
// sum of squares is reordered (it differs from another order by ~1e-16
// relative).  Each rounding to bf16 is one round to nearest even of the fp64
// value, and the division is a correctly rounded fp64 division.
//
// One wave per token row: all loads of the row first (CH 16-byte pieces per
// lane, CH = ceil(hidden / 512), a template argument so that registers are
// sized for the row at hand), the sum of squares reduced across the wave,
// then the row written back.  Batches of at most kNormRowTokens rows spread
// each row over a workgroup instead (rmsnorm_row_kernel).  The traffic is 2 bytes per element for each of
// x, residual in, out and residual out; at the measured rate the per-element
// fp64 arithmetic and roundings (a few dozen instructions), not the bytes,
// set the time.
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

__device__ __forceinline__ uint16_t half_of(const u32x4& v, int e) {
  const uint32_t w = v[e >> 1];
  return (uint16_t)((e & 1) ? (w >> 16) : (w & 0xffffu));
}

// The 8 values of one 16-byte piece: r = bf16(x + residual) (r = x without
// a residual), their squares added to ss.
__device__ __forceinline__ u32x4 add_piece(u32x4 x, u32x4 res, bool has_res, double& ss) {
  u32x4 out;
#pragma unroll
  for (int e2 = 0; e2 < 4; ++e2) {
    uint16_t r[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint16_t xb = half_of(x, 2 * e2 + h);
      r[h] = has_res ? rne_bf16((double)bf_to_f(xb) + (double)bf_to_f(half_of(res, 2 * e2 + h)))
                     : xb;
      const double rv = (double)bf_to_f(r[h]);
      ss += rv * rv;
    }
    out[e2] = (uint32_t)r[0] | ((uint32_t)r[1] << 16);
  }
  return out;
}

// out = bf16(w * bf16(r / s)) (no weight: bf16(r / s)) for the 8 values of a piece.
__device__ __forceinline__ u32x4 norm_piece(u32x4 r, u32x4 w, bool has_w, double s) {
  u32x4 o;
#pragma unroll
  for (int e2 = 0; e2 < 4; ++e2) {
    uint16_t ob[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int e = 2 * e2 + h;
      const uint16_t yb = rne_bf16((double)bf_to_f(half_of(r, e)) / s);
      ob[h] = has_w ? rne_bf16((double)bf_to_f(half_of(w, e)) * (double)bf_to_f(yb)) : yb;
    }
    o[e2] = (uint32_t)ob[0] | ((uint32_t)ob[1] << 16);
  }
  return o;
}

template <int CH>
__global__ __launch_bounds__(256) void rmsnorm_hidden_kernel(NormArgs a) {
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
      if (a.w) wr[c] = ld16(a.w + 8 * i);
    }
  }
  double ss = 0.0;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int i = lane + 64 * c;
    if (i < nc) rr[c] = add_piece(xr[c], rr[c], a.res != nullptr, ss);
  }
  ss = wave_sum(ss);
  const double s = sqrt(ss / (double)a.hidden + a.eps);
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int i = lane + 64 * c;
    if (i < nc) {
      st16(a.out + row + 8 * i, norm_piece(rr[c], wr[c], a.w != nullptr, s));
      if (a.res) st16(a.res + row + 8 * i, rr[c]);
    }
  }
}

// Up to kNormRowTokens rows: one workgroup per row and one 16-byte piece per
// thread, so a row's serial fp64 work is one piece deep instead of hidden/512
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
    st16(a.out + row + 8 * i, norm_piece(rr, wr, a.w != nullptr, s));
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
