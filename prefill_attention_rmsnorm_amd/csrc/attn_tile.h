// MFMA tile machinery shared by the prefill and verify attention kernels.
//
// A workgroup owns up to 128 query rows of one (sequence, kv head) and walks
// the keys in tiles of 64.  Per tile:
//   S^T[key][query] = K . Q'^T   (v_mfma_f32_32x32x16_bf16, K from LDS as A,
//                                 Q' kept in registers as B)
//   online softmax per query column (one query per lane pair, exp2 domain)
//   O^T[d][query] += V^T . P^T   (V^T from LDS as A, P^T from registers as B)
// Orienting the products with queries on the MFMA column axis keeps every
// per-query quantity (running max, sum, rescale) inside one lane, so the only
// cross-lane step per tile is one swap between lane l and l^32.
//
// K rows are read into the A operand in a permuted order sigma(i) chosen so
// that the S^T registers of a lane hold 8 consecutive keys per 16-key chunk:
// P^T can then be fed to the PV product straight from registers.
#pragma once

#include "qa_device.h"

namespace qa {

constexpr int kKStride = 272;   // bytes per K row in LDS (256 + 16 pad)
constexpr int kVtStride = 144;  // bytes per V^T row in LDS (64 keys*2 + 16 pad)
constexpr int kKTileBytes = kKeyTile * kKStride;          // 17408
constexpr int kVtTileBytes = kHeadDim * kVtStride;        // 18432
constexpr int kStageBytes = kKTileBytes + kVtTileBytes;   // 35840

// A-operand row i of the QK product holds key sigma(i) of a 32-key block:
// S^T register r of lane half h2 then holds key 16*(r/8) + 8*h2 + r%8.
__device__ __forceinline__ int sigma_row(int i) {
  return 16 * (i >> 4) + 8 * ((i >> 2) & 1) + 4 * ((i >> 3) & 1) + (i & 3);
}
__device__ __forceinline__ int key_of_reg(int r, int h2) {
  return 16 * (r >> 3) + 8 * h2 + (r & 7);
}

// Staging of one 64-key tile: global -> registers -> LDS.  NT threads; K stays row-major (padded), V is
// transposed to V^T[d][key] on the way into LDS.
template <int NT>
struct TileStage {
  static constexpr int KPER = 1024 / NT;  // 16-byte K chunks per thread
  static constexpr int VUNITS = 256 / NT; // (4 keys x 8 dims) units per thread
  u32x4 k[KPER];
  u32x4 v[VUNITS * 4];

  // Rows at or beyond kend are loaded from row kend-1 instead (a written
  // slot; such keys are masked, so their V rows are multiplied by p = 0).
  // The loads are unconditional so that all of them are in flight at once.
  __device__ __forceinline__ void load(const uint16_t* kbase,
                                       const uint16_t* vbase, int64_t sp,
                                       int kv0, int kend, int tid) {
#pragma unroll
    for (int i = 0; i < KPER; ++i) {
      const int ci = tid + NT * i;
      const int key = min(kv0 + (ci >> 4), kend - 1), c = ci & 15;
      k[i] = ld16(kbase + (size_t)key * sp + 8 * c);
    }
#pragma unroll
    for (int u = 0; u < VUNITS; ++u) {
      const int ui = tid + NT * u;
      const int kg = ui & 15, c = ui >> 4;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = min(kv0 + 4 * kg + i, kend - 1);
        v[4 * u + i] = ld16(vbase + (size_t)key * sp + 8 * c);
      }
    }
  }

  __device__ __forceinline__ void store(unsigned char* stage, int tid) const {
    unsigned char* ks = stage;
    unsigned char* vs = stage + kKTileBytes;
#pragma unroll
    for (int i = 0; i < KPER; ++i) {
      const int ci = tid + NT * i;
      st16(ks + (ci >> 4) * kKStride + (ci & 15) * 16, k[i]);
    }
#pragma unroll
    for (int u = 0; u < VUNITS; ++u) {
      const int ui = tid + NT * u;
      const int kg = ui & 15, c = ui >> 4;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t w0 = v[4 * u + 0][e >> 1], w1 = v[4 * u + 1][e >> 1];
        const uint32_t w2 = v[4 * u + 2][e >> 1], w3 = v[4 * u + 3][e >> 1];
        u32x2 pr;
        if (e & 1) {
          pr[0] = (w0 >> 16) | (w1 & 0xffff0000u);
          pr[1] = (w2 >> 16) | (w3 & 0xffff0000u);
        } else {
          pr[0] = (w0 & 0xffffu) | (w1 << 16);
          pr[1] = (w2 & 0xffffu) | (w3 << 16);
        }
        *reinterpret_cast<u32x2*>(vs + (8 * c + e) * kVtStride + 8 * kg) = pr;
      }
    }
  }
};

// Per-wave attention state for 32 query columns.
struct WaveAttn {
  f32x16 o[4];  // O^T, d-block db: rows d = 32*db + 8*(r/4) + 4*h2 + r%4
  float m;      // running max (log2 domain), per query (lane)
  float lsum;   // running sum of this lane's half of the keys

  __device__ __forceinline__ void init() {
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
    m = -__builtin_inff();
    lsum = 0.f;
  }

  // One 64-key tile held in LDS `stage`.  qb: Q'^T operand (8 k-steps).
  // Keys kv0 + x are masked when kv0 + x >= kmax_excl or kv0 + x > p.
  __device__ __forceinline__ void tile(const unsigned char* stage,
                                       const u32x4 (&qb)[8], int kv0,
                                       bool need_mask, int p, int kmax_excl,
                                       int j, int h2) {
    const unsigned char* ks = stage;
    const unsigned char* vs = stage + kKTileBytes;
    const int srow = sigma_row(j);
    f32x16 s0, s1;
#pragma unroll
    for (int r = 0; r < 16; ++r) { s0[r] = 0.f; s1[r] = 0.f; }
#pragma unroll
    for (int kstep = 0; kstep < 8; ++kstep) {
      const int off = (16 * kstep + 8 * h2) * 2;
      const u32x4 a0 = *reinterpret_cast<const u32x4*>(ks + srow * kKStride + off);
      const u32x4 a1 = *reinterpret_cast<const u32x4*>(ks + (32 + srow) * kKStride + off);
      s0 = mfma32x32x16(a0, qb[kstep], s0);
      s1 = mfma32x32x16(a1, qb[kstep], s1);
    }
    const float ninf = -__builtin_inff();
    if (need_mask) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int k0 = kv0 + key_of_reg(r, h2);
        const int k1 = k0 + 32;
        if (k0 > p || k0 >= kmax_excl) s0[r] = ninf;
        if (k1 > p || k1 >= kmax_excl) s1[r] = ninf;
      }
    }
    float mt = ninf;
#pragma unroll
    for (int r = 0; r < 16; ++r) mt = fmaxf(mt, fmaxf(s0[r], s1[r]));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float mn = fmaxf(m, mt);
    if (__any(mn > m)) {
      // a row with no visible key so far keeps m = -inf; exp2 of -inf is 0
      const float alpha = (mn == ninf) ? 1.f : __builtin_amdgcn_exp2f(m - mn);
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
      lsum *= alpha;
      m = mn;
    }
    const float mu = (m == ninf) ? 0.f : m;
    u32x4 pb[4];
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const float p0 = __builtin_amdgcn_exp2f(s0[r] - mu);
      const float p1 = __builtin_amdgcn_exp2f(s0[r + 1] - mu);
      const float p2 = __builtin_amdgcn_exp2f(s1[r] - mu);
      const float p3 = __builtin_amdgcn_exp2f(s1[r + 1] - mu);
      lsum += (p0 + p1) + (p2 + p3);
      pb[r >> 3][(r & 7) >> 1] = pack_bf16x2(p0, p1);
      pb[2 + (r >> 3)][(r & 7) >> 1] = pack_bf16x2(p2, p3);
    }
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const u32x4 va = *reinterpret_cast<const u32x4*>(
            vs + (32 * db + j) * kVtStride + (16 * c + 8 * h2) * 2);
        o[db] = mfma32x32x16(va, pb[c], o[db]);
      }
    }
  }
};

// q' = RoPE(RMSNorm(q)) * qscale for the lane's half of one query row, packed
// as the B operand of the QK product.  Lane half h2 owns dims
// d = 16*kstep + 8*h2 + e; pairs (d, d+64) are kstep and kstep+4 of the same
// lane.  cs[i] = (cos, sin) of the query's angle for pair i (64 entries).
__device__ __forceinline__ void q_prologue(const uint16_t* qrow, bool valid,
                                           const float2* cs,
                                           const uint16_t* wq, float eps,
                                           float qscale, int h2,
                                           u32x4 (&qb)[8]) {
  float x[8][8];
  float ss = 0.f;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    u32x4 v = {0u, 0u, 0u, 0u};
    if (valid) v = ld16(qrow + 16 * ks + 8 * h2);
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) {
      x[ks][2 * e2] = bf_lo(v[e2]);
      x[ks][2 * e2 + 1] = bf_hi(v[e2]);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) ss += x[ks][e] * x[ks][e];
  }
  ss += __shfl_xor(ss, 32);
  const float rinv = 1.0f / sqrtf(ss * (1.0f / 128.0f) + eps);
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    float w0[8], w1[8];
    if (wq) {
      const u32x4 a = ld16(wq + 16 * ks + 8 * h2);
      const u32x4 b = ld16(wq + 64 + 16 * ks + 8 * h2);
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        w0[2 * e2] = bf_lo(a[e2]); w0[2 * e2 + 1] = bf_hi(a[e2]);
        w1[2 * e2] = bf_lo(b[e2]); w1[2 * e2 + 1] = bf_hi(b[e2]);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) { w0[e] = 1.f; w1[e] = 1.f; }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float2 t = valid ? cs[16 * ks + 8 * h2 + e] : make_float2(1.f, 0.f);
      const float y0 = x[ks][e] * rinv * w0[e];
      const float y1 = x[ks + 4][e] * rinv * w1[e];
      x[ks][e] = (y0 * t.x - y1 * t.y) * qscale;
      x[ks + 4][e] = (y1 * t.x + y0 * t.y) * qscale;
    }
  }
#pragma unroll
  for (int ks = 0; ks < 8; ++ks)
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2)
      qb[ks][e2] = pack_bf16x2(x[ks][2 * e2], x[ks][2 * e2 + 1]);
}

}  // namespace qa
