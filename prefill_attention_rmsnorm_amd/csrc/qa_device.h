// Device helpers shared by the gfx950 kernels of libqa.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qa_internal.h"

namespace qa {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---- bf16 <-> fp32 -------------------------------------------------------
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf_to_f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// Two floats -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2 r;
  r[0] = (__bf16)a;
  r[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, r);
}

// fp64 -> bf16 bits with a single round-to-nearest-even (no fp32 step, which
// would round twice).  Normal values keep 8 significant bits; below 2^-126
// the quantum is the bf16 subnormal step 2^-133.  NaN -> quiet NaN.
__device__ __forceinline__ uint16_t f64_to_bf16_rne(double x) {
  if (x != x) return (uint16_t)(0x7FC0u | (signbit(x) ? 0x8000u : 0u));
  if (x == 0.0 || __builtin_isinf(x))
    return (uint16_t)(__float_as_uint((float)x) >> 16);
  int e;
  (void)frexp(x, &e);  // x = m * 2^e, 0.5 <= |m| < 1
  int qexp = e - 8;
  if (qexp < -133) qexp = -133;
  double r = ldexp(rint(ldexp(x, -qexp)), qexp);  // rint: ties to even
  // r is bf16-representable (or +-2^128, which converts to +-inf: overflow)
  return (uint16_t)(__float_as_uint((float)r) >> 16);
}

// acc + a.lo*b.lo + a.hi*b.hi over packed bf16 pairs (v_dot2c_f32_bf16).
// The operands are taken as scalars on purpose: bit-casting an element of an
// ext_vector (v[e]) inside __builtin_bit_cast loses the element index in this
// compiler and silently reads element 0.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                         __builtin_bit_cast(bf16x2, b), acc, false);
}

// ---- MFMA -----------------------------------------------------------------
// D(32x32 fp32) += A(32x16 bf16) * B(16x32 bf16).  Lane l holds
// A[l%32][8*(l/32) .. +7], B[8*(l/32) .. +7][l%32], and D column l%32, rows
// 8*(r/4) + 4*(l/32) + r%4 for register r.
__device__ __forceinline__ f32x16 mfma32x32x16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(
      __builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// D(16x16 fp32) += A(16x32 bf16) * B(32x16 bf16).  Lane l holds
// A[l%16][8*(l/16) .. +7], B[8*(l/16) .. +7][l%16], and D rows 4*(l/16) + r
// of column l%16 for register r.
typedef float f32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(
      __builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// D(16x16 fp32) += A(16x16 bf16) * B(16x16 bf16).  Lane l holds
// A[l%16][4*(l/16) .. +3] and B[4*(l/16) .. +3][l%16] as two bf16 pairs
// each, and D rows 4*(l/16) + r of column l%16 for register r.
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f32x4 mfma16x16x16(u32x2 a, u32x2 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                   __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
}

// ---- cross-lane ------------------------------------------------------------
// Max / sum over the lanes l, l^16, l^32, l^48 (one lane of each 16-lane
// row); every lane gets the result.  permlane32_swap(x, x) returns x and x of
// the lane 32 away; permlane16_swap(x, x) the same for the lane 16 away.
__device__ __forceinline__ float rows4_max(float x) {
  auto t = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(t[0]), __uint_as_float(t[1]));
  t = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(t[0]), __uint_as_float(t[1]));
}
__device__ __forceinline__ float rows4_add(float x) {
  auto t = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(t[0]) + __uint_as_float(t[1]);
  t = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(t[0]) + __uint_as_float(t[1]);
}

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL,
                                                    0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm(1,0,3,2)
constexpr int kDppXor2 = 0x4E;        // quad_perm(2,3,0,1)
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7-i within 8
constexpr int kDppMirror = 0x140;     // lane i <-> 15-i within 16

// Sum over the 16 lanes of a DPP row; every lane of the row gets the total.
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp<kDppXor1>(x);
  x += dpp<kDppXor2>(x);
  x += dpp<kDppHalfMirror>(x);
  x += dpp<kDppMirror>(x);
  return x;
}

__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, dpp<kDppXor1>(x));
  x = fmaxf(x, dpp<kDppXor2>(x));
  x = fmaxf(x, dpp<kDppHalfMirror>(x));
  x = fmaxf(x, dpp<kDppMirror>(x));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}
__device__ __forceinline__ double wave_sum(double x) {
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// ---- memory ---------------------------------------------------------------
__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void st16(void* p, u32x4 v) {
  *reinterpret_cast<u32x4*>(p) = v;
}

// cos/sin of an fp64 angle in fp32: Cody-Waite reduction by 2*pi in fp64,
// then the fp32 library sincos on |r| <= pi (query side, where the result is
// rounded to bf16 anyway).
__device__ __forceinline__ void sincos_reduced(double a, float* s, float* c) {
  const double k = rint(a * 0.15915494309189535);
  double r = fma(-k, 6.283185307179586, a);
  r = fma(-k, 2.4492935982947064e-16, r);
  sincosf((float)r, s, c);
}

// Log-sum-exp merge of n_split partial rows (m: max in log2 units, l: sum,
// o: unnormalised output) for 4 consecutive dims of one row, in split order.
// load(s, m, l, o) fetches split s's values; loads are issued CH splits at a
// time (slots past n_split load split n_split - 1 again and count as empty)
// so that a merge costs one memory round trip per CH splits, with no branch
// between the loads or in the arithmetic.  A split with m = -inf is empty
// and adds exactly zero (its o is not read into the sums).  Both merge paths
// (the merge kernel and decode's in-launch merge) run this one piece of
// arithmetic and differ only in how they load.
struct MergeOut {
  float m, l;
  float4 o;
};
// IG rows at a time: load(j, s, m, l, o) fetches split s of row j; the loads
// of all IG rows and CH splits are issued before any arithmetic.  Per row
// the arithmetic is the same as for a single row.
template <int CH, int IG, class Load>
__device__ __forceinline__ void merge_splits_n(int n_split, Load&& load, MergeOut (&r)[IG]) {
  const float ninf = -__builtin_inff();
#pragma unroll
  for (int j = 0; j < IG; ++j) {
    r[j].m = ninf;
    r[j].l = 0.f;
    r[j].o = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  for (int s0 = 0; s0 < n_split; s0 += CH) {
    float mv[IG][CH], lv[IG][CH];
    float4 ov[IG][CH];
#pragma unroll
    for (int j = 0; j < IG; ++j)
#pragma unroll
      for (int c = 0; c < CH; ++c) load(j, min(s0 + c, n_split - 1), mv[j][c], lv[j][c], ov[j][c]);
#pragma unroll
    for (int j = 0; j < IG; ++j) {
#pragma unroll
      for (int c = 0; c < CH; ++c)
        if (s0 + c >= n_split) mv[j][c] = ninf;  // (a select, not a branch)
      float mc = ninf;
#pragma unroll
      for (int c = 0; c < CH; ++c) mc = fmaxf(mc, mv[j][c]);
      const float mn = fmaxf(r[j].m, mc);
      const float alpha = (r[j].m == ninf) ? 0.f : __builtin_amdgcn_exp2f(r[j].m - mn);
      r[j].l *= alpha;
      r[j].o.x *= alpha; r[j].o.y *= alpha; r[j].o.z *= alpha; r[j].o.w *= alpha;
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        const bool empty = mv[j][c] == ninf;
        const float wgt = empty ? 0.f : __builtin_amdgcn_exp2f(mv[j][c] - mn);
        const float4 o = empty ? make_float4(0.f, 0.f, 0.f, 0.f) : ov[j][c];
        r[j].l += wgt * (empty ? 0.f : lv[j][c]);
        r[j].o.x += wgt * o.x; r[j].o.y += wgt * o.y;
        r[j].o.z += wgt * o.z; r[j].o.w += wgt * o.w;
      }
      r[j].m = mn;
    }
  }
}
template <int CH, class Load>
__device__ __forceinline__ MergeOut merge_splits(int n_split, Load&& load) {
  MergeOut r[1];
  merge_splits_n<CH, 1>(
      n_split, [&](int, int s, float& m, float& l, float4& o) { load(s, m, l, o); }, r);
  return r[0];
}

// The merged row as bf16 output (4 dims) and natural-log LSE; a row with no
// visible key (l = 0), or one the caller marks bad, becomes zeros.
__device__ __forceinline__ void store_merged(const MergeOut& mo, bool bad, uint16_t* orow4,
                                             float* lse) {
  const bool good = !bad && mo.l > 0.f;
  const float inv = good ? 1.0f / mo.l : 0.f;
  u32x2 pr = {0u, 0u};
  if (good) {
    pr[0] = pack_bf16x2(mo.o.x * inv, mo.o.y * inv);
    pr[1] = pack_bf16x2(mo.o.z * inv, mo.o.w * inv);
  }
  *reinterpret_cast<u32x2*>(orow4) = pr;
  if (lse) *lse = good ? (mo.m + __log2f(mo.l)) * kLn2 : 0.f;
}

__device__ __forceinline__ void flag_error(int* err, int bits) {
  __hip_atomic_fetch_or(err, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---- the K-side prologue ----------------------------------------------------
// One wave turns one 128-element k row into k' = RoPE(RMSNorm(k)) in fp64 and
// rounds it once to bf16.  Lane i owns elements i and i+64 (a rotation pair).
// c, s: cos/sin of pos * inv_freq[i] in fp64.  The operation order is that of
// the definition: x / sqrt(mean(x^2) + eps) * w, then x1 c - x2 s, x2 c + x1 s.
__device__ __forceinline__ void kprime_pair(uint16_t k_lo, uint16_t k_hi,
                                            double w_lo, double w_hi,
                                            double eps, double c, double s,
                                            uint16_t* out_lo,
                                            uint16_t* out_hi) {
#pragma clang fp contract(off)
  double x0 = (double)bf_to_f(k_lo), x1 = (double)bf_to_f(k_hi);
  double ss = wave_sum(x0 * x0 + x1 * x1);  // exact for bf16 inputs
  double r = sqrt(ss / 128.0 + eps);
  double y0 = x0 / r * w_lo;
  double y1 = x1 / r * w_hi;
  double o0 = y0 * c - y1 * s;
  double o1 = y1 * c + y0 * s;
  *out_lo = f64_to_bf16_rne(o0);
  *out_hi = f64_to_bf16_rne(o1);
}

}  // namespace qa
