// MFMA tile machinery shared by the prefill and verify attention kernels.
//
// A workgroup owns up to 128 query rows of one (sequence, kv head) and walks
// the keys in tiles of 64.  Per tile:
//   S^T[key][query] = K . Q'^T   (v_mfma_f32_32x32x16_bf16, K from LDS as A,
//                                 Q' kept in registers as B)
//   online softmax per query column (exp2 domain)
//   O^T[d][query] += V^T . P^T   (V^T read from LDS with the transposing
//                                 ds_read_b64_tr_b16 as A, P^T from registers)
// Orienting the products with queries on the MFMA column axis keeps every
// per-query quantity inside one lane pair (l, l^32).
//
// K and V tiles travel HBM/L2 -> LDS with buffer_load ... lds (no register
// staging).  Rows at or beyond the tile's key limit fall outside the buffer
// descriptor's range and arrive as zeros; their scores are masked, so they
// add 0 * 0.  Each 16-byte chunk of a 256-byte row is stored at an
// XOR-swizzled position so that the MFMA operand reads hit distinct banks:
//   K: chunk c of row r at position c ^ (r & 15)
//   V: chunk c of row r at position c ^ (4 * (r & 3))
#pragma once

#include "qa_device.h"

namespace qa {

constexpr int kRowBytes = kHeadDim * 2;                   // 256
constexpr int kKTileBytes = kKeyTile * kRowBytes;         // 16384
constexpr int kStageBytes = 2 * kKTileBytes;              // K then V: 32768
constexpr float kRescaleSlack = 8.0f;  // log2 units a stale max may lag by

typedef __attribute__((address_space(3))) void lds_void;
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// A-operand row i of the QK product holds key sigma(i) of a 32-key block:
// S^T register r of lane half h2 then holds key 16*(r/8) + 8*h2 + r%8, which
// is the k index order the PV product wants for P^T.
__device__ __forceinline__ int sigma_row(int i) {
  return 16 * (i >> 4) + 8 * ((i >> 2) & 1) + 4 * ((i >> 3) & 1) + (i & 3);
}

// 16 bytes per lane from a buffer into LDS at lds + 16 * lane.  (Kept as a
// non-template function: called straight from a kernel template, the builtin
// makes the host pass drop the launch stubs of later instantiations.)
__device__ __forceinline__ void buffer_load_lds16(__amdgpu_buffer_rsrc_t r, void* lds,
                                                  uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, voff, 0, 0, 0);
}

// Global -> LDS copy of one 64-key K/V tile by the NW waves of a workgroup.
// A stage is 32 one-KiB pieces (16 of K, 16 of V), each 4 rows; wave w moves
// pieces w, w + NW, ...  Lane L of a piece lands at LDS byte 16*L of it.
template <int NW>
struct TileLoader {
  static constexpr int NI = 16 / NW;  // K (and V) pieces per wave
  uint32_t koff[NI], voff[NI];        // per-lane byte offsets from the tile's row 0
  int w;                              // wave index (uniform)

  __device__ __forceinline__ void init(int wave, int lane, int64_t sp) {
    w = wave;
    const uint32_t spb = (uint32_t)sp * 2u;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int q = w + NW * i;
      const int r = 4 * q + (lane >> 4);
      const int pos = lane & 15;
      koff[i] = (uint32_t)r * spb + (uint32_t)((pos ^ (r & 15)) << 4);
      voff[i] = (uint32_t)r * spb + (uint32_t)((pos ^ ((r & 3) << 2)) << 4);
    }
  }

  // Keys kv0 .. kv0+63 of the rows at kbase/vbase (element stride sp); keys at
  // or beyond kend read as zero.
  __device__ __forceinline__ void load(const uint16_t* kbase, const uint16_t* vbase,
                                       int64_t sp, int kv0, int kend,
                                       unsigned char* stage) const {
    const int nrows = min(max(kend - kv0, 0), kKeyTile);
    // < 2^31 since sp <= kMaxStridePos; readfirstlane keeps the descriptor
    // in SGPRs (a VALU min/max would otherwise force a waterfall loop)
    const int nrec = __builtin_amdgcn_readfirstlane(nrows * (int)sp * 2);
    const size_t off = (size_t)kv0 * (size_t)sp;
    const __amdgpu_buffer_rsrc_t rk =
        __builtin_amdgcn_make_buffer_rsrc((void*)(kbase + off), 0, nrec, 0x00020000);
    const __amdgpu_buffer_rsrc_t rv =
        __builtin_amdgcn_make_buffer_rsrc((void*)(vbase + off), 0, nrec, 0x00020000);
#pragma unroll
    for (int i = 0; i < NI; ++i)
      buffer_load_lds16(rk, stage + (w + NW * i) * 1024, koff[i]);
#pragma unroll
    for (int i = 0; i < NI; ++i)
      buffer_load_lds16(rv, stage + kKTileBytes + (w + NW * i) * 1024, voff[i]);
  }
};

// Wait until this wave's tile copies have landed in LDS.
__device__ __forceinline__ void wait_tile_loads() {
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
}

// Per-wave attention state for 32 query columns.
struct WaveAttn {
  f32x16 o[4];  // O^T, d-block db: rows d = 32*db + 8*(r/4) + 4*h2 + r%4
  float m;      // running (possibly stale) max, log2 domain, per query
  float lsum;   // sum of this lane's half of the bf16-rounded probabilities
  uint32_t kaddr[8];  // LDS byte offsets of this lane's K operand per k-step
  uint32_t vaddr[4];  // LDS byte offsets of this lane's V^T piece per d-block

  __device__ __forceinline__ void init(int lane) {
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
    m = -__builtin_inff();
    lsum = 0.f;
    const int j = lane & 31, h2 = lane >> 5;
    // K operand: row sigma(j) (+32 for the second 32-key block), dims
    // 16*kstep + 8*h2 .. +7 = logical chunk 2*kstep + h2.
    const int sj = sigma_row(j);
    const int y = (sj & 15) ^ h2;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      kaddr[ks] = (uint32_t)(sj * kRowBytes + ((y ^ (2 * ks)) << 4));
    // V^T operand through ds_read_b64_tr_b16: in each 16-lane group, lane s
    // reads 4 dims of key row (base + s/4); the transpose hands lane i of the
    // group dim (i) of those 4 consecutive keys.  Group g16 covers dims
    // 16*(g16&1) .. +15 of the d-block and keys 8*(g16>>1) .. +3 (+4 for the
    // second read).
    const int g16 = lane >> 4, s = lane & 15, e = s >> 2, r4 = s & 3;
    const int x = 2 * (g16 & 1) + (r4 >> 1);
    const uint32_t vb = (uint32_t)((8 * (g16 >> 1) + e) * kRowBytes + 16 * x + 8 * (r4 & 1));
#pragma unroll
    for (int db = 0; db < 4; ++db) vaddr[db] = vb + 64u * (uint32_t)(db ^ e);
  }

  // One 64-key tile held in LDS `stage`.  qb: Q'^T operand (8 k-steps).
  // When need_mask, key kv0 + x counts only if kv0 + x <= lim_abs, where
  // lim_abs = min(query position, last valid key).
  __device__ __forceinline__ void tile(const unsigned char* stage,
                                       const u32x4 (&qb)[8], int kv0,
                                       bool need_mask, int lim_abs, int h2) {
    const unsigned char* ks = stage;
    const unsigned char* vs = stage + kKTileBytes;
    f32x16 s0, s1;
#pragma unroll
    for (int r = 0; r < 16; ++r) { s0[r] = 0.f; s1[r] = 0.f; }
#pragma unroll
    for (int kstep = 0; kstep < 8; ++kstep) {
      const u32x4 a0 = *reinterpret_cast<const u32x4*>(ks + kaddr[kstep]);
      const u32x4 a1 = *reinterpret_cast<const u32x4*>(ks + 32 * kRowBytes + kaddr[kstep]);
      s0 = mfma32x32x16(a0, qb[kstep], s0);
      s1 = mfma32x32x16(a1, qb[kstep], s1);
    }
    const float ninf = -__builtin_inff();
    if (need_mask) {
      const int lim = lim_abs - kv0 - 8 * h2;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kr = 16 * (r >> 3) + (r & 7);
        s0[r] = (kr > lim) ? ninf : s0[r];
        s1[r] = (kr + 32 > lim) ? ninf : s1[r];
      }
    }
    float mt = ninf;
#pragma unroll
    for (int r = 0; r < 16; ++r) mt = fmaxf(mt, fmaxf(s0[r], s1[r]));
    // The max is refreshed only when a score passes the stale one by more
    // than kRescaleSlack, so p <= 2^kRescaleSlack and the O rescale is rare.
    if (__any(mt > m + kRescaleSlack)) {
      const float mn = fmaxf(m, fmaxf(mt, __shfl_xor(mt, 32)));
      // a row with no visible key so far keeps m = -inf (o and lsum are 0)
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
      pb[r >> 3][(r & 7) >> 1] = pack_bf16x2(__builtin_amdgcn_exp2f(s0[r] - mu),
                                             __builtin_amdgcn_exp2f(s0[r + 1] - mu));
      pb[2 + (r >> 3)][(r & 7) >> 1] = pack_bf16x2(__builtin_amdgcn_exp2f(s1[r] - mu),
                                                   __builtin_amdgcn_exp2f(s1[r + 1] - mu));
    }
    constexpr uint32_t kOnes = 0x3F803F80u;  // bf16 (1, 1)
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i) lsum = dot2_bf16(pb[c][i], kOnes, lsum);
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const s16x4 t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4*)(vs + vaddr[db] + 16 * c * kRowBytes));
        const s16x4 t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4*)(vs + vaddr[db] + (16 * c + 4) * kRowBytes));
        const u32x2 w0 = __builtin_bit_cast(u32x2, t0);
        const u32x2 w1 = __builtin_bit_cast(u32x2, t1);
        u32x4 va;
        va[0] = w0[0]; va[1] = w0[1]; va[2] = w1[0]; va[3] = w1[1];
        o[db] = mfma32x32x16(va, pb[c], o[db]);
      }
    }
  }
};

// q' = RoPE(RMSNorm(q)) * qscale for the lane's half of one query row, packed
// as the B operand of the QK product.  Lane half h2 owns dims
// d = 16*kstep + 8*h2 + e; pairs (d, d+64) are kstep and kstep+4 of the same
// lane.  cs[i] = (cos, sin) of the query's angle for pair i (64 entries).
// load() only issues the reads, so a kernel can start other loads before the
// values are needed; compute() consumes them.
struct QPrologue {
  u32x4 q[8];     // raw q, dims 16*ks + 8*h2 .. +7
  float4 cs[16];  // (cos, sin) of pairs 16*ks + 8*h2 + 2u, +1 at [4*ks + u]
  u32x4 w[8];     // norm weights: [ks] dims 16*ks + 8*h2.., [4+ks] dims 64 + ..

  __device__ __forceinline__ void load(const uint16_t* qrow, bool valid,
                                       const float2* csrow, const uint16_t* wq,
                                       int h2) {
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      q[ks] = u32x4{0u, 0u, 0u, 0u};
      if (valid) q[ks] = ld16(qrow + 16 * ks + 8 * h2);
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        cs[4 * ks + u] = make_float4(1.f, 0.f, 1.f, 0.f);
        if (valid)
          cs[4 * ks + u] = reinterpret_cast<const float4*>(csrow + 16 * ks + 8 * h2)[u];
      }
    const uint32_t one2 = 0x3F803F80u;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      w[ks] = u32x4{one2, one2, one2, one2};
      if (wq) w[ks] = ld16(wq + 64 * (ks >> 2) + 16 * (ks & 3) + 8 * h2);
    }
  }

  __device__ __forceinline__ void compute(float eps, float qscale,
                                          u32x4 (&qb)[8]) const {
    float x[8][8];
    float ss = 0.f;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        x[ks][2 * e2] = bf_lo(q[ks][e2]);
        x[ks][2 * e2 + 1] = bf_hi(q[ks][e2]);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) ss += x[ks][e] * x[ks][e];
    }
    ss += __shfl_xor(ss, 32);
    const float rinv = 1.0f / sqrtf(ss * (1.0f / 128.0f) + eps);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float4 c4 = cs[4 * ks + (e >> 1)];
        const float c = (e & 1) ? c4.z : c4.x;
        const float sn = (e & 1) ? c4.w : c4.y;
        const uint32_t wa = w[ks][e >> 1], wb = w[4 + ks][e >> 1];
        const float w0 = (e & 1) ? bf_hi(wa) : bf_lo(wa);
        const float w1 = (e & 1) ? bf_hi(wb) : bf_lo(wb);
        const float y0 = x[ks][e] * rinv * w0;
        const float y1 = x[ks + 4][e] * rinv * w1;
        x[ks][e] = (y0 * c - y1 * sn) * qscale;
        x[ks + 4][e] = (y1 * c + y0 * sn) * qscale;
      }
    }
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2)
        qb[ks][e2] = pack_bf16x2(x[ks][2 * e2], x[ks][2 * e2 + 1]);
  }
};

}  // namespace qa
