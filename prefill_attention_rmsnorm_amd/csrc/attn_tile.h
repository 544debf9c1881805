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

typedef __attribute__((address_space(3))) void lds_void;
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// max(a, b, c) with one v_max3_f32 (IEEE maxNum on quiet values; inputs here
// are finite scores or -inf).
__device__ __forceinline__ float max3_f32(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

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

// Global -> LDS copy of a 64-key K or V tile by the NW waves of a workgroup.
// A tile is 16 one-KiB pieces of 4 rows; wave w moves pieces w, w + NW, ...
// Lane L of a piece lands at LDS byte 16*L of it.
template <int NW>
struct TileLoader {
  static constexpr int NI = 16 / NW;  // pieces per wave and tile
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

  // Rows kv0 .. kv0+63 of the row array at base (element stride sp) into the
  // LDS tile dst; rows at or beyond kend read as zero.
  __device__ __forceinline__ void load(const uint16_t* base, int64_t sp, int kv0,
                                       int kend, unsigned char* dst,
                                       const uint32_t (&off)[NI]) const {
    const int nrows = min(max(kend - kv0, 0), kKeyTile);
    // < 2^31 since sp <= kMaxStridePos; readfirstlane keeps the descriptor
    // in SGPRs (a VALU min/max would otherwise force a waterfall loop)
    const int nrec = __builtin_amdgcn_readfirstlane(nrows * (int)sp * 2);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(base + (size_t)kv0 * (size_t)sp), 0, nrec, 0x00020000);
#pragma unroll
    for (int i = 0; i < NI; ++i)
      buffer_load_lds16(rs, dst + (w + NW * i) * 1024, off[i]);
  }
  __device__ __forceinline__ void load_k(const uint16_t* kbase, int64_t sp, int kv0,
                                         int kend, unsigned char* dst) const {
    load(kbase, sp, kv0, kend, dst, koff);
  }
  __device__ __forceinline__ void load_v(const uint16_t* vbase, int64_t sp, int kv0,
                                         int kend, unsigned char* dst) const {
    load(vbase, sp, kv0, kend, dst, voff);
  }
};

// Wait until this wave's tile copies have landed in LDS.
__device__ __forceinline__ void wait_tile_loads() {
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
}

// The four LDS tiles of a workgroup: K and V, double-buffered.  They must be
// four distinct __shared__ arrays of kKTileBytes: only then can the compiler
// see that reads of one buffer do not depend on a copy in flight into
// another (it would otherwise wait for the copy before every read).
struct AttnLds {
  unsigned char* k0;
  unsigned char* k1;
  unsigned char* v0;
  unsigned char* v1;
};

// Scores above the block's reference max by more than this (log2 units), or
// an output that large, send the block to the exact-max path.
constexpr float kSumLimit = 0x1p96f;
constexpr float kOutLimit = 0x1p126f;

// Per-wave attention state for 32 query columns.
//
// Softmax with a reference max fixed per workgroup: m is the row max over
// the first tile processed, and every later tile uses p = exp2(s - m) with
// no rescaling of O.  Softmax is invariant to the shift, so this is the same
// quantity as with the running max as long as nothing overflows; a later
// score far above m shows up as a huge row sum, and the caller then redoes
// the block with the exact row max (where p <= 1 everywhere).
struct WaveAttn {
  f32x16 o[4];  // O^T, d-block db: rows d = 32*db + 8*(r/4) + 4*h2 + r%4
  float m;      // reference max (log2 domain), per query
  float lsum;   // sum of this lane's half of the probabilities (fp32, before rounding)
  uint32_t kb;  // LDS byte offset of this lane's K operand at k-step 0
  uint32_t vb;  // LDS byte offset of this lane's V^T piece at d-block 0

  __device__ __forceinline__ void reset() {
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
    lsum = 0.f;
  }

  __device__ __forceinline__ void init(int lane) {
    reset();
    m = 0.f;
    const int j = lane & 31, h2 = lane >> 5;
    // K operand: row sigma(j) (+32 for the second 32-key block), dims
    // 16*kstep + 8*h2 .. +7 = logical chunk 2*kstep + h2, stored at chunk
    // (2*kstep + h2) ^ (row & 15); the k-step enters as an XOR of 32*kstep.
    const int sj = sigma_row(j);
    kb = (uint32_t)(sj * kRowBytes + ((((sj & 15) ^ h2)) << 4));
    // V^T operand through ds_read_b64_tr_b16: in each 16-lane group, lane s
    // reads 4 dims of key row (base + s/4); the transpose hands lane i of the
    // group dim (i) of those 4 consecutive keys.  Group g16 covers dims
    // 16*(g16&1) .. +15 of the d-block and keys 8*(g16>>1) .. +3 (+4 for the
    // second read).  Logical chunk 4*db + x of row r sits at chunk
    // (4*db + x) ^ (4*(r&3)); the d-block enters as an XOR of 64*db.
    const int g16 = lane >> 4, s = lane & 15, e = s >> 2, r4 = s & 3;
    const int x = 2 * (g16 & 1) + (r4 >> 1);
    vb = (uint32_t)((8 * (g16 >> 1) + e) * kRowBytes + 64 * e + 16 * x + 8 * (r4 & 1));
  }

  // K operand of one k-step for keys 0-31 (a0) and 32-63 (a1).
  __device__ __forceinline__ static void read_k(const unsigned char* kt, uint32_t kbt,
                                                int kstep, u32x4& a0, u32x4& a1) {
    const uint32_t off = kbt ^ (32u * kstep);
    a0 = *reinterpret_cast<const u32x4*>(kt + off);
    a1 = *reinterpret_cast<const u32x4*>(kt + off + 32 * kRowBytes);
  }

  // V^T operand of d-block db, 16-key chunk c (two transposing reads of 4
  // keys each, landing in the two halves of one operand).
  __device__ __forceinline__ static u32x4 read_vt(const unsigned char* vt, uint32_t vbt,
                                                  int db, int c) {
    const uint32_t vo = vbt ^ (64u * db);
    const s16x4 t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4*)(vt + vo + 16 * c * kRowBytes));
    const s16x4 t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4*)(vt + vo + (16 * c + 4) * kRowBytes));
    return __builtin_bit_cast(u32x4, __builtin_shufflevector(t0, t1, 0, 1, 2, 3, 4, 5, 6, 7));
  }

  // Re-derive the LDS offsets in each tile (one XOR per use) rather than
  // keeping a dozen of them live across the loop.
  __device__ __forceinline__ void offsets(uint32_t& kbt, uint32_t& vbt) const {
    kbt = kb;
    vbt = vb;
    asm volatile("" : "+v"(kbt), "+v"(vbt));
  }

  // S^T of the 64 keys of the K tile kt: s0 keys 0-31, s1 keys 32-63;
  // register r of lane half h2 holds key 16*(r/8) + 8*h2 + r%8 (+32 in s1).
  __device__ __forceinline__ static void qk(const unsigned char* kt, uint32_t kbt,
                                            const u32x4 (&qb)[8], f32x16& s0, f32x16& s1) {
    u32x4 ka[8];  // ring of 4 k-steps, reads two k-steps ahead of use
    read_k(kt, kbt, 0, ka[0], ka[1]);
    read_k(kt, kbt, 1, ka[2], ka[3]);
    read_k(kt, kbt, 2, ka[4], ka[5]);
    read_k(kt, kbt, 3, ka[6], ka[7]);
#pragma unroll
    for (int r = 0; r < 16; ++r) { s0[r] = 0.f; s1[r] = 0.f; }
#pragma unroll
    for (int kstep = 0; kstep < 8; kstep += 2) {
      const int u = (kstep & 3) * 2;
      s0 = mfma32x32x16(ka[u], qb[kstep], s0);
      s1 = mfma32x32x16(ka[u + 1], qb[kstep], s1);
      s0 = mfma32x32x16(ka[u + 2], qb[kstep + 1], s0);
      s1 = mfma32x32x16(ka[u + 3], qb[kstep + 1], s1);
      if (kstep + 4 < 8) {
        read_k(kt, kbt, kstep + 4, ka[u], ka[u + 1]);
        read_k(kt, kbt, kstep + 5, ka[u + 2], ka[u + 3]);
      }
    }
  }

  // Masks keys kv0 + x > lim_abs (lim_abs = min(query position, last valid
  // key)) to -inf.
  __device__ __forceinline__ static void mask(f32x16& s0, f32x16& s1, int kv0,
                                              int lim_abs, int h2) {
    const float ninf = -__builtin_inff();
    const int lim = lim_abs - kv0 - 8 * h2;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kr = 16 * (r >> 3) + (r & 7);
      s0[r] = (kr > lim) ? ninf : s0[r];
      s1[r] = (kr + 32 > lim) ? ninf : s1[r];
    }
  }

  // Row max of a tile's (masked) scores, both lane halves combined.
  __device__ __forceinline__ static float row_max(const f32x16& s0, const f32x16& s1) {
    float mt = -__builtin_inff();
#pragma unroll
    for (int r = 0; r < 16; ++r) mt = max3_f32(mt, s0[r], s1[r]);
    return fmaxf(mt, __shfl_xor(mt, 32));
  }

  // Scores -> bf16 P^T (pb[c]: keys 16c .. 16c+15) with the reference max.
  // The row sum adds the fp32 probabilities before their rounding to bf16
  // (a pairwise tree per tile, plain fp32 adds).  A v_dot2 over the packed
  // values gives the same sum within the rounding, but it does not overlap
  // MFMAs on the same SIMD (an MFMA wave and a dot2 wave sharing one take
  // the sum of their times), while fp32 adds do.
  template <bool MASK>
  __device__ __forceinline__ void probs(f32x16& s0, f32x16& s1, int kv0, int lim_abs,
                                        int h2, u32x4 (&pb)[4]) {
    if (MASK) mask(s0, s1, kv0, lim_abs, h2);
    float part[8];
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const float e0 = __builtin_amdgcn_exp2f(s0[r] - m);
      const float e1 = __builtin_amdgcn_exp2f(s0[r + 1] - m);
      const float e2 = __builtin_amdgcn_exp2f(s1[r] - m);
      const float e3 = __builtin_amdgcn_exp2f(s1[r + 1] - m);
      pb[r >> 3][(r & 7) >> 1] = pack_bf16x2(e0, e1);
      pb[2 + (r >> 3)][(r & 7) >> 1] = pack_bf16x2(e2, e3);
      part[r >> 1] = (e0 + e1) + (e2 + e3);
    }
    lsum += ((part[0] + part[1]) + (part[2] + part[3])) +
            ((part[4] + part[5]) + (part[6] + part[7]));
  }

  // QK of the next tile (K tile kn, into sn) interleaved with the
  // probabilities of the current tile (sc -> pb): the MFMAs run while the
  // VALU computes exponentials.
  template <bool MASK>
  __device__ __forceinline__ void qk_probs(const unsigned char* kn, uint32_t kbt,
                                           const u32x4 (&qb)[8], f32x16& sn0, f32x16& sn1,
                                           f32x16& sc0, f32x16& sc1, int kv0, int lim_abs,
                                           int h2, u32x4 (&pb)[4]) {
    qk(kn, kbt, qb, sn0, sn1);
    probs<MASK>(sc0, sc1, kv0, lim_abs, h2, pb);
    // 16 MFMAs, 16 LDS reads and ~110 VALU: one MFMA, one read, seven VALU
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 7, 0);
    }
  }

  // O^T += V^T . P^T with the V tile vt.
  __device__ __forceinline__ void pv(const unsigned char* vt, uint32_t vbt,
                                     const u32x4 (&pb)[4]) {
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      u32x4 va[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) va[c] = read_vt(vt, vbt, db, c);
#pragma unroll
      for (int c = 0; c < 4; ++c) o[db] = mfma32x32x16(va[c], pb[c], o[db]);
    }
  }

  // P.V of one tile (V tile vt, probabilities pb) followed by the QK product
  // of the next K tile kn into s0/s1, with LDS reads issued two groups of
  // MFMAs ahead: for a wave that is alone on the matrix core, nothing else
  // hides the read latency.
  template <bool QK>
  __device__ __forceinline__ void pv_qk(const unsigned char* vt, uint32_t vbt,
                                        const u32x4 (&pb)[4], const unsigned char* kn,
                                        uint32_t kbt, const u32x4 (&qb)[8], f32x16& s0,
                                        f32x16& s1) {
    u32x4 va[8], ka[8];
#pragma unroll
    for (int c = 0; c < 4; ++c) va[c] = read_vt(vt, vbt, 0, c);
#pragma unroll
    for (int c = 0; c < 4; ++c) va[4 + c] = read_vt(vt, vbt, 1, c);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int u = (db & 1) * 4;
#pragma unroll
      for (int c = 0; c < 4; ++c) o[db] = mfma32x32x16(va[u + c], pb[c], o[db]);
      if (db + 2 < 4) {
#pragma unroll
        for (int c = 0; c < 4; ++c) va[u + c] = read_vt(vt, vbt, db + 2, c);
      } else if (QK) {
        read_k(kn, kbt, 2 * (db - 2), ka[4 * (db - 2)], ka[4 * (db - 2) + 1]);
        read_k(kn, kbt, 2 * (db - 2) + 1, ka[4 * (db - 2) + 2], ka[4 * (db - 2) + 3]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (!QK) return;
#pragma unroll
    for (int r = 0; r < 16; ++r) { s0[r] = 0.f; s1[r] = 0.f; }
#pragma unroll
    for (int kstep = 0; kstep < 8; kstep += 2) {
      const int u = (kstep & 3) * 2;
      s0 = mfma32x32x16(ka[u], qb[kstep], s0);
      s1 = mfma32x32x16(ka[u + 1], qb[kstep], s1);
      s0 = mfma32x32x16(ka[u + 2], qb[kstep + 1], s0);
      s1 = mfma32x32x16(ka[u + 3], qb[kstep + 1], s1);
      if (kstep + 4 < 8) {
        read_k(kn, kbt, kstep + 4, ka[u], ka[u + 1]);
        read_k(kn, kbt, kstep + 5, ka[u + 2], ka[u + 3]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // Whether this lane's results might have overflowed the reference max
  // (row sum or |O| too large, or not finite).
  __device__ __forceinline__ bool overflowed() const {
    const float lt = lsum + __shfl_xor(lsum, 32);
    float om = 0.f;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) om = fmaxf(om, fabsf(o[db][r]));
    return !(lt < kSumLimit) || !(om < kOutLimit);
  }
};

// First loads of attend_pass: K and V of the tile at kbeg, K of the next.
template <int NW>
__device__ __forceinline__ void load_first(const TileLoader<NW>& ld, const AttnLds& lds,
                                           const uint16_t* kbase, const uint16_t* vbase,
                                           int64_t sp, int kbeg, int kend) {
  ld.load_k(kbase, sp, kbeg, kend, lds.k0);
  ld.load_v(vbase, sp, kbeg, kend, lds.v0);
  if (kbeg + kKeyTile < kend) ld.load_k(kbase, sp, kbeg + kKeyTile, kend, lds.k1);
}

// One pass over keys kbeg .. kend-1 in 64-key tiles.  Tile kt's K sits in
// k(kt&1) and its V in v(kt&1); while tile kt is consumed, K of tile kt+2
// and V of tile kt+1 load, and the QK product of tile kt+1 runs interleaved
// with the exponentials of tile kt.  The first n_unmasked tiles hold no key
// beyond any row's limit; the rest (the diagonal) are masked: key kv0 + x
// counts only if kv0 + x <= lim_abs.  With SET_M the reference max is taken
// from the first tile, otherwise st.m is used as given.  The caller issued
// load_first().  Ends with a barrier.
template <bool SET_M, int NW>
__device__ __forceinline__ void attend_pass(WaveAttn& st, const TileLoader<NW>& ld,
                                            const AttnLds& lds, const uint16_t* kbase,
                                            const uint16_t* vbase, int64_t sp, int kbeg,
                                            int kend, int n_unmasked, const u32x4 (&qb)[8],
                                            int lim_abs, int h2) {
  const int n_kt = (kend - kbeg + kKeyTile - 1) / kKeyTile;
  uint32_t kbt, vbt;
  st.offsets(kbt, vbt);
  wait_tile_loads();
  __syncthreads();
  f32x16 sc0, sc1, sn0, sn1;
  WaveAttn::qk(lds.k0, kbt, qb, sc0, sc1);
  if (SET_M) {
    f32x16 t0 = sc0, t1 = sc1;
    if (n_unmasked == 0) WaveAttn::mask(t0, t1, kbeg, lim_abs, h2);
    st.m = WaveAttn::row_max(t0, t1);
  }
  __syncthreads();  // every wave has read K tile 0 before it is reloaded
  int kt = 0;
  // steady state: two unmasked tiles per iteration, each naming its buffers
  for (; kt + 2 < n_kt && kt + 2 <= n_unmasked; kt += 2) {
    const int kv0 = kbeg + kt * kKeyTile;
    u32x4 pb[4];
    ld.load_k(kbase, sp, kv0 + 2 * kKeyTile, kend, lds.k0);
    ld.load_v(vbase, sp, kv0 + kKeyTile, kend, lds.v1);
    st.qk_probs<false>(lds.k1, kbt, qb, sn0, sn1, sc0, sc1, kv0, lim_abs, h2, pb);
    st.pv(lds.v0, vbt, pb);
    sc0 = sn0;
    sc1 = sn1;
    wait_tile_loads();
    __syncthreads();
    if (kt + 3 < n_kt) ld.load_k(kbase, sp, kv0 + 3 * kKeyTile, kend, lds.k1);
    ld.load_v(vbase, sp, kv0 + 2 * kKeyTile, kend, lds.v0);
    st.qk_probs<false>(lds.k0, kbt, qb, sn0, sn1, sc0, sc1, kv0 + kKeyTile, lim_abs, h2, pb);
    st.pv(lds.v1, vbt, pb);
    sc0 = sn0;
    sc1 = sn1;
    wait_tile_loads();
    __syncthreads();
  }
  // the rest (the diagonal; usually one or two tiles), masked, one tile per
  // iteration and not interleaved: probabilities, PV, then QK of the next
  // tile into the same score registers
  const unsigned char* knext = (kt & 1) ? lds.k0 : lds.k1;  // K of tile kt+1
  unsigned char* kload = (kt & 1) ? lds.k1 : lds.k0;        // for K of tile kt+2
  const unsigned char* vcur = (kt & 1) ? lds.v1 : lds.v0;   // V of tile kt
  unsigned char* vload = (kt & 1) ? lds.v0 : lds.v1;        // for V of tile kt+1
  for (; kt < n_kt; ++kt) {
    const int kv0 = kbeg + kt * kKeyTile;
    if (kt + 2 < n_kt) ld.load_k(kbase, sp, kv0 + 2 * kKeyTile, kend, kload);
    if (kt + 1 < n_kt) ld.load_v(vbase, sp, kv0 + kKeyTile, kend, vload);
    u32x4 pb[4];
    st.probs<true>(sc0, sc1, kv0, lim_abs, h2, pb);
    st.pv(vcur, vbt, pb);
    if (kt + 1 < n_kt) WaveAttn::qk(knext, kbt, qb, sc0, sc1);
    wait_tile_loads();
    __syncthreads();
    const unsigned char* kt_ = knext;
    knext = kload;
    kload = const_cast<unsigned char*>(kt_);
    const unsigned char* vt_ = vcur;
    vcur = vload;
    vload = const_cast<unsigned char*>(vt_);
  }
}

// Exact row max over keys kbeg .. kend-1 (QK only, K tiles double-buffered).
template <int NW>
__device__ __forceinline__ float exact_row_max(const WaveAttn& st, const TileLoader<NW>& ld,
                                               const AttnLds& lds, const uint16_t* kbase,
                                               int64_t sp, int kbeg, int kend,
                                               const u32x4 (&qb)[8], int lim_abs, int h2) {
  const int n_kt = (kend - kbeg + kKeyTile - 1) / kKeyTile;
  uint32_t kbt, vbt;
  st.offsets(kbt, vbt);
  float mx = -__builtin_inff();
  ld.load_k(kbase, sp, kbeg, kend, lds.k0);
  for (int kt = 0; kt < n_kt; ++kt) {
    const int kv0 = kbeg + kt * kKeyTile;
    wait_tile_loads();
    __syncthreads();
    const unsigned char* cur = (kt & 1) ? lds.k1 : lds.k0;
    if (kt + 1 < n_kt) ld.load_k(kbase, sp, kv0 + kKeyTile, kend, (kt & 1) ? lds.k0 : lds.k1);
    f32x16 s0, s1;
    WaveAttn::qk(cur, kbt, qb, s0, s1);
    WaveAttn::mask(s0, s1, kv0, lim_abs, h2);
    mx = fmaxf(mx, WaveAttn::row_max(s0, s1));
    __syncthreads();  // reads of `cur` done before it is reloaded
  }
  return mx;
}

// ---- four-stage K/V ring ----------------------------------------------------
//
// For a run of a few tiles that streams from HBM, most copies of the run can
// be in flight before the first tile is used.  Tile t's K sits in LDS buffer
// t & 3 and its V likewise.  The copies go out in the order K0 V0 K1 V1 K2 V2
// (ring_first: six tiles, which with a wave's few other loads stays within
// the 63 memory operations its counter can track, so issue does not stall)
// and then, at step j, K(j+3) and V(j+3), each into the buffer its previous
// tile (K(j-1), V(j-1)) left by step j-1; copies of tiles past the run read
// as zeros and are issued all the same, so at the top of step j exactly three
// tiles' copies were issued after the ones it needs (K(j+1), V(j)), and
// before the first step five after K0.  The waits count this wave's own
// copies; the barrier after them makes every wave's pieces visible and ends
// every read of the buffers about to be refilled.
struct RingLds {
  unsigned char *k0, *k1, *k2, *k3, *v0, *v1, *v2, *v3;
};
// The buffers by compile-time index, so that the compiler sees which LDS
// array each read and each copy touches (a copy in flight into one buffer
// then does not hold up reads of another).
template <int I>
__device__ __forceinline__ unsigned char* ring_k(const RingLds& r) {
  if constexpr (I == 0) return r.k0;
  else if constexpr (I == 1) return r.k1;
  else if constexpr (I == 2) return r.k2;
  else return r.k3;
}
template <int I>
__device__ __forceinline__ unsigned char* ring_v(const RingLds& r) {
  if constexpr (I == 0) return r.v0;
  else if constexpr (I == 1) return r.v1;
  else if constexpr (I == 2) return r.v2;
  else return r.v3;
}

// Wait until at most N of this wave's vector memory operations are in flight
// (s_waitcnt: vmcnt in bits 3:0 and 15:14, expcnt and lgkmcnt left at their
// maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt holds 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// A workgroup barrier that orders LDS only: this wave's LDS accesses drain
// (lgkmcnt) and the "memory" clobber keeps the compiler from moving LDS
// accesses across it.  __syncthreads() would also wait for every copy into
// LDS in flight, which the ring keeps in flight on purpose.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int NW>
__device__ __forceinline__ void ring_first(const TileLoader<NW>& ld, const RingLds& r,
                                           const uint16_t* kbase, const uint16_t* vbase,
                                           int64_t sp, int kbeg, int kend) {
  ld.load_k(kbase, sp, kbeg, kend, r.k0);
  ld.load_v(vbase, sp, kbeg, kend, r.v0);
  ld.load_k(kbase, sp, kbeg + kKeyTile, kend, r.k1);
  ld.load_v(vbase, sp, kbeg + kKeyTile, kend, r.v1);
  ld.load_k(kbase, sp, kbeg + 2 * kKeyTile, kend, r.k2);
  ld.load_v(vbase, sp, kbeg + 2 * kKeyTile, kend, r.v2);
}

// Step j (J4 = j & 3) of the ring: the probabilities of tile j interleaved
// with the QK product of tile j+1, then P.V of tile j.  Tile j is unmasked.
template <int J4, int NW>
__device__ __forceinline__ void ring_step(WaveAttn& st, const TileLoader<NW>& ld,
                                          const RingLds& r, const uint16_t* kbase,
                                          const uint16_t* vbase, int64_t sp, int kbeg,
                                          int kend, int j, uint32_t kbt, uint32_t vbt,
                                          const u32x4 (&qb)[8], f32x16& sc0, f32x16& sc1,
                                          int h2) {
  wait_vmcnt<3 * TileLoader<NW>::NI>();  // K(j+1), V(j)
  lds_barrier();
  ld.load_k(kbase, sp, kbeg + (j + 3) * kKeyTile, kend, ring_k<(J4 + 3) & 3>(r));
  ld.load_v(vbase, sp, kbeg + (j + 3) * kKeyTile, kend, ring_v<(J4 + 3) & 3>(r));
  f32x16 sn0, sn1;
  u32x4 pb[4];
  st.qk_probs<false>(ring_k<(J4 + 1) & 3>(r), kbt, qb, sn0, sn1, sc0, sc1, 0, 0, h2, pb);
  st.pv(ring_v<J4>(r), vbt, pb);
  sc0 = sn0;
  sc1 = sn1;
}

// One pass over keys kbeg .. kend-1 with the ring (the caller issued
// ring_first).  Every tile but the last lies wholly below kend and at or
// below every query's position (no mask); the last is masked when
// last_masked.  With SET_M the reference max is taken from tile 0.  Ends
// with every copy landed and a full barrier.
template <bool SET_M, int NW>
__device__ __forceinline__ void attend_ring_pass(WaveAttn& st, const TileLoader<NW>& ld,
                                                 const RingLds& r, const uint16_t* kbase,
                                                 const uint16_t* vbase, int64_t sp,
                                                 int kbeg, int kend, bool last_masked,
                                                 const u32x4 (&qb)[8], int lim_abs, int h2) {
  const int n_kt = (kend - kbeg + kKeyTile - 1) / kKeyTile;
  uint32_t kbt, vbt;
  st.offsets(kbt, vbt);
  wait_vmcnt<5 * TileLoader<NW>::NI>();  // K0
  lds_barrier();
  f32x16 sc0, sc1;
  WaveAttn::qk(r.k0, kbt, qb, sc0, sc1);
  if (SET_M) {
    f32x16 t0 = sc0, t1 = sc1;
    if (n_kt == 1 && last_masked) WaveAttn::mask(t0, t1, kbeg, lim_abs, h2);
    st.m = WaveAttn::row_max(t0, t1);
  }
  int j = 0;
  for (; j + 4 <= n_kt - 1; j += 4) {
    ring_step<0>(st, ld, r, kbase, vbase, sp, kbeg, kend, j, kbt, vbt, qb, sc0, sc1, h2);
    ring_step<1>(st, ld, r, kbase, vbase, sp, kbeg, kend, j + 1, kbt, vbt, qb, sc0, sc1, h2);
    ring_step<2>(st, ld, r, kbase, vbase, sp, kbeg, kend, j + 2, kbt, vbt, qb, sc0, sc1, h2);
    ring_step<3>(st, ld, r, kbase, vbase, sp, kbeg, kend, j + 3, kbt, vbt, qb, sc0, sc1, h2);
  }
  if (j < n_kt - 1) {
    ring_step<0>(st, ld, r, kbase, vbase, sp, kbeg, kend, j, kbt, vbt, qb, sc0, sc1, h2);
    ++j;
    if (j < n_kt - 1) {
      ring_step<1>(st, ld, r, kbase, vbase, sp, kbeg, kend, j, kbt, vbt, qb, sc0, sc1, h2);
      ++j;
      if (j < n_kt - 1) {
        ring_step<2>(st, ld, r, kbase, vbase, sp, kbeg, kend, j, kbt, vbt, qb, sc0, sc1, h2);
        ++j;
      }
    }
  }
  // the last tile: nothing left to load ahead, so every copy is waited for
  wait_tile_loads();
  __syncthreads();
  u32x4 pb[4];
  if (last_masked) st.probs<true>(sc0, sc1, kbeg + j * kKeyTile, lim_abs, h2, pb);
  else st.probs<false>(sc0, sc1, kbeg + j * kKeyTile, lim_abs, h2, pb);
  const unsigned char* vl = (j & 3) == 0 ? r.v0 : (j & 3) == 1 ? r.v1 : (j & 3) == 2 ? r.v2 : r.v3;
  st.pv(vl, vbt, pb);
  __syncthreads();
}

// attend_ring_pass with the exact-max fallback (the double-buffered pass over
// the ring's first two K and V buffers).  The caller issued ring_first().
template <int NW>
__device__ __forceinline__ void attend_ring(WaveAttn& st, const TileLoader<NW>& ld,
                                            const RingLds& r, const uint16_t* kbase,
                                            const uint16_t* vbase, int64_t sp, int kbeg,
                                            int kend, bool last_masked, const u32x4 (&qb)[8],
                                            int lim_abs, int h2) {
  attend_ring_pass<true>(st, ld, r, kbase, vbase, sp, kbeg, kend, last_masked, qb, lim_abs, h2);
  if (__syncthreads_or(st.overflowed())) {
    const AttnLds lds{r.k0, r.k1, r.v0, r.v1};
    const int n_unmasked = (kend - kbeg) / kKeyTile;
    st.m = exact_row_max(st, ld, lds, kbase, sp, kbeg, kend, qb, lim_abs, h2);
    st.reset();
    load_first(ld, lds, kbase, vbase, sp, kbeg, kend);
    attend_pass<false>(st, ld, lds, kbase, vbase, sp, kbeg, kend, n_unmasked, qb, lim_abs, h2);
  }
}

// Attention of this wave's 32 query rows over keys kbeg .. kend-1 (see
// attend_pass), with the exact-max fallback.  The caller issued load_first().
template <int NW>
__device__ __forceinline__ void attend(WaveAttn& st, const TileLoader<NW>& ld,
                                       const AttnLds& lds, const uint16_t* kbase,
                                       const uint16_t* vbase, int64_t sp, int kbeg, int kend,
                                       int n_unmasked, const u32x4 (&qb)[8], int lim_abs,
                                       int h2) {
  attend_pass<true>(st, ld, lds, kbase, vbase, sp, kbeg, kend, n_unmasked, qb, lim_abs, h2);
  if (__syncthreads_or(st.overflowed())) {
    st.m = exact_row_max(st, ld, lds, kbase, sp, kbeg, kend, qb, lim_abs, h2);
    st.reset();
    load_first(ld, lds, kbase, vbase, sp, kbeg, kend);
    attend_pass<false>(st, ld, lds, kbase, vbase, sp, kbeg, kend, n_unmasked, qb, lim_abs,
                       h2);
  }
}

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

  // q and norm weights only; the cos/sin then come from cs_from_lds().
  __device__ __forceinline__ void load_qw(const uint16_t* qrow, bool valid,
                                          const uint16_t* wq, int h2) {
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      q[ks] = u32x4{0u, 0u, 0u, 0u};
      if (valid) q[ks] = ld16(qrow + 16 * ks + 8 * h2);
    }
    const uint32_t one2 = 0x3F803F80u;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      w[ks] = u32x4{one2, one2, one2, one2};
      if (wq) w[ks] = ld16(wq + 64 * (ks >> 2) + 16 * (ks & 3) + 8 * h2);
    }
  }

  // cos/sin of the lane's pairs from an LDS copy of the block's table rows:
  // row tl (512 bytes, 32 chunks of two pairs) holds chunk c at chunk
  // position c ^ (tl & 31).
  __device__ __forceinline__ void cs_from_lds(const unsigned char* rows, int tl, int h2) {
    const unsigned char* row = rows + tl * 512;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int c = 8 * ks + 4 * h2 + u;
        cs[4 * ks + u] = *reinterpret_cast<const float4*>(row + 16 * (c ^ (tl & 31)));
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
