// Prompt prefill on gfx950: K/V prologue + causal GQA flash attention.
//
// "dryft-flash-infer" agent guide, Where the wins are: prefill is a large share
// of the time at prompts of 512-2048 tokens; RMSNorm and rotary embedding are
// fused; the cache is preallocated and strided.  Kernel 1 writes the cache
// (fp64 K prologue, one RNE to bf16) and a cos/sin table for the queries;
// kernel 2 normalises and rotates q while loading it and runs the MFMA flash
// loop over the cache.
#include <climits>

#include "attn_tile.h"
#include "qa.h"

namespace qa {

// The XCDs a launch's workgroups are dealt over (round-robin by block index);
// the attention grid keeps one q-tile counter per XCD in the workspace header
// (ints 1..8, after the error word).
constexpr int kPrefillXcds = 8;
static_assert((1 + kPrefillXcds) * sizeof(int) <= kWsHeader, "counters fit the header");

// One wave per token: cos/sin of its angles, then k' and v of every KV head.
// Eight lanes per KV head and eight heads at a time: lane group gh (lanes
// 8gh .. 8gh+7) holds head gh, lane sub = lane & 7 its rotation pairs
// i = 8*sub + e (e < 8), i.e. dims 8*sub .. +7 and 64 + 8*sub .. +7, read as
// two 16-byte pieces.  The head's sum of squares is then a 3-step reduction
// inside the group (exact in fp64 for bf16 inputs of moderate range, so its
// order does not matter), and the arithmetic per element is the fp64
// sequence x / r * w, rotation, one round to bf16.  A token whose position is
// out of range writes no cache slot.
// k' and v of one KV head into its cache slot: lane sub holds dims
// 8*sub .. +7 (ka, va) and 64 + 8*sub .. +7 (kb, vb); the eight lanes of the
// head reduce the sum of squares in fp64.
__device__ __forceinline__ void kv_head(uint16_t* ck, uint16_t* cv, int sub, u32x4 ka,
                                        u32x4 kb, u32x4 va, u32x4 vb, const double (&w0)[8],
                                        const double (&w1)[8], const double (&cs_c)[8],
                                        const double (&cs_s)[8], double eps, bool active) {
  double x0[8], x1[8];
#pragma unroll
  for (int e2 = 0; e2 < 4; ++e2) {
    x0[2 * e2] = bf_lo(ka[e2]); x0[2 * e2 + 1] = bf_hi(ka[e2]);
    x1[2 * e2] = bf_lo(kb[e2]); x1[2 * e2 + 1] = bf_hi(kb[e2]);
  }
  u32x4 oa, ob;
  {
#pragma clang fp contract(off)
    double ss = 0.0;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss += x0[e] * x0[e] + x1[e] * x1[e];
    ss += __shfl_xor(ss, 1);
    ss += __shfl_xor(ss, 2);
    ss += __shfl_xor(ss, 4);
    const double r = sqrt(ss / 128.0 + eps);
    uint16_t o0[8], o1[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const double y0 = x0[e] / r * w0[e];
      const double y1 = x1[e] / r * w1[e];
      o0[e] = f64_to_bf16_rne(y0 * cs_c[e] - y1 * cs_s[e]);
      o1[e] = f64_to_bf16_rne(y1 * cs_c[e] + y0 * cs_s[e]);
    }
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) {
      oa[e2] = (uint32_t)o0[2 * e2] | ((uint32_t)o0[2 * e2 + 1] << 16);
      ob[e2] = (uint32_t)o1[2 * e2] | ((uint32_t)o1[2 * e2 + 1] << 16);
    }
  }
  if (active) {
    st16(ck + 8 * sub, oa);
    st16(ck + 64 + 8 * sub, ob);
    st16(cv + 8 * sub, va);
    st16(cv + 64 + 8 * sub, vb);
  }
}

__device__ __forceinline__ void bf16x8_to_f64(u32x4 w, double (&d)[8]) {
#pragma unroll
  for (int e2 = 0; e2 < 4; ++e2) {
    d[2 * e2] = bf_lo(w[e2]);
    d[2 * e2 + 1] = bf_hi(w[e2]);
  }
}

__global__ __launch_bounds__(256) void kv_prologue_kernel(PrefillArgs a,
                                                          RopeFreq f) {
  __shared__ double2 s_cs[4][kHalf];  // per wave: (cos, sin) of the 64 pairs
  if (blockIdx.x == 0 && threadIdx.x < kPrefillXcds) a.tile_ctr[threadIdx.x] = 0;  // for the attention grid
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wv;
  if (t >= a.total_tokens) return;
  const int gh = lane >> 3, sub = lane & 7;

  // ---- every load first: the work of a token is a few short dependent
  // steps, so the memory latency is paid once per wave, not once per step.
  const int pos = a.positions[t];
  const double invf = f.inv_freq[lane];  // (a lane-indexed kernel-argument load)
  const int cuv = lane <= a.n_seq ? a.cu_seqlens[lane] : INT_MAX;
  const u32x4 one8 = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
  const uint16_t* kwp = a.k_norm_w ? a.k_norm_w : a.q;
  const u32x4 kwa = ld16(kwp + 8 * sub), kwb = ld16(kwp + 64 + 8 * sub);
  const bool kact = gh < a.n_kv_heads;
  const size_t ksrc = (size_t)t * a.kv_tok_stride + (size_t)(kact ? gh : 0) * kHeadDim;
  const u32x4 ka = ld16(a.k + ksrc + 8 * sub), kb = ld16(a.k + ksrc + 64 + 8 * sub);
  const u32x4 va = ld16(a.v + ksrc + 8 * sub), vb = ld16(a.v + ksrc + 64 + 8 * sub);

  // ---- cos/sin of the token's 64 angles (fp64), one pair per lane
  {
    double sn = 0.0, cn = 1.0;
    sincos((double)pos * invf, &sn, &cn);
    a.cs[(size_t)t * kHalf + lane] = make_float2((float)cn, (float)sn);
    s_cs[wv][lane] = make_double2(cn, sn);
  }

  // ---- sequence owning token t: the number of boundaries cu[1..n_seq] at
  // or below t (one ballot for up to 63 sequences, else a binary search)
  int seq;
  if (a.n_seq < 64) {
    seq = __popcll(__ballot(lane >= 1 && lane <= a.n_seq && cuv <= t));
  } else {
    int lo = 0, hi = a.n_seq;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (a.cu_seqlens[mid] <= t) lo = mid; else hi = mid;
    }
    seq = lo;
  }
  seq = min(seq, a.n_seq - 1);
  const int c0 = a.cu_seqlens[seq], c1 = a.cu_seqlens[seq + 1];
  if (!(c0 <= t && t < c1 && c1 - c0 <= a.max_seqlen)) {
    if (lane == 0) flag_error(a.err, QA_DEVERR_SEQLENS);
    return;
  }
  if (pos < 0 || pos >= a.c.capacity) {
    if (lane == 0) flag_error(a.err, QA_DEVERR_POSITION);
    return;
  }

  __builtin_amdgcn_wave_barrier();  // s_cs of this wave written
  double cs_c[8], cs_s[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const double2 v = s_cs[wv][8 * sub + e];
    cs_c[e] = v.x;
    cs_s[e] = v.y;
  }

  // ---- k' and v of every KV head (eight at a time)
  double kw0[8], kw1[8];
  bf16x8_to_f64(a.k_norm_w ? kwa : one8, kw0);
  bf16x8_to_f64(a.k_norm_w ? kwb : one8, kw1);
  const size_t row0 = (size_t)seq * a.c.sb + (size_t)pos * a.c.sp;
  kv_head(a.c.k + row0 + (size_t)gh * a.c.sh, a.c.v + row0 + (size_t)gh * a.c.sh, sub, ka,
          kb, va, vb, kw0, kw1, cs_c, cs_s, a.eps, kact);
  for (int g0 = 8; g0 < a.n_kv_heads; g0 += 8) {
    const int g = g0 + gh;
    const bool act = g < a.n_kv_heads;
    const size_t src = (size_t)t * a.kv_tok_stride + (size_t)(act ? g : 0) * kHeadDim;
    kv_head(a.c.k + row0 + (size_t)g * a.c.sh, a.c.v + row0 + (size_t)g * a.c.sh, sub,
            ld16(a.k + src + 8 * sub), ld16(a.k + src + 64 + 8 * sub),
            ld16(a.v + src + 8 * sub), ld16(a.v + src + 64 + 8 * sub), kw0, kw1, cs_c,
            cs_s, a.eps, act);
  }
}

// ---------------------------------------------------------------------------
// Attention: workgroup = 8 waves = 256 query rows = G heads x (256/G) tokens
// of one sequence and KV head, all sharing every K/V tile.  Waves 0-3 (group
// A) and 4-7 (group B) sit one of each on every SIMD and run the same tile
// sequence half a tile apart: each tile takes two barrier-separated phases,
// and in every phase one group issues the MFMA work (P.V of the previous
// tile, then Q.K of the next) while the other group computes the
// exponentials of its current scores.  The matrix core thus always has a
// wave feeding it while the softmax runs on the vector ALUs.
//
// Phase 2k (even) starts the copies of K tile k+1 and V tile k (into the
// buffers whose previous contents were last read two phases earlier); phase
// 2k+1 (odd) ends with every wave waiting for its copies.  Only group B
// issues copies: its even phases are its exponential phases, which have
// slack, while a copy issued by the MFMA group delays its first MFMA.  Group A runs
// M(k) in phase 2k and V(k) in 2k+1; group B one phase later; both pass
// the same number of barriers.
//   M(k): O += V(k-1)^T . P(k-1)^T (k >= 1);  S = K(k) . Q'^T (k < n_kt)
//   V(k): P(k) = exp2(S - m) as bf16, masked on the diagonal tiles

template <int PAR>
__device__ __forceinline__ void pp_loads(const TileLoader<4>& ld, const AttnLds& lds,
                                         const uint16_t* kbase, const uint16_t* vbase,
                                         int64_t sp, int kend, int kk, int n_kt) {
  // even phase 2kk: K(kk+1) -> k[(kk+1)&1], V(kk) -> v[kk&1]; PAR = kk & 1
  if (kk + 1 < n_kt) ld.load_k(kbase, sp, (kk + 1) * kKeyTile, kend, PAR ? lds.k0 : lds.k1);
  if (kk < n_kt) ld.load_v(vbase, sp, kk * kKeyTile, kend, PAR ? lds.v1 : lds.v0);
}

// Keep a phase's results on its own side of the barrier that ends it: the
// barrier orders memory only, and the compiler would otherwise sink pure
// ALU work (the exponentials, or MFMAs) into the next phase, where it would
// serialise with the other kind of work instead of overlapping the other
// group's.
__device__ __forceinline__ void pin(const u32x4 (&pb)[4], float x) {
  asm volatile("" ::"v"(pb[0]), "v"(pb[1]), "v"(pb[2]), "v"(pb[3]), "v"(x));
}
__device__ __forceinline__ void pin(const f32x16& a, const f32x16& b) {
  asm volatile("" ::"v"(a), "v"(b));
}
__device__ __forceinline__ void pin(const f32x16 (&o)[4]) {
  asm volatile("" ::"v"(o[0]), "v"(o[1]), "v"(o[2]), "v"(o[3]));
}

// The barrier between ping-pong phases.  __syncthreads() fences workgroup
// memory, and the fence waits for every copy into LDS still in flight, which
// would expose the copy latency in the phase that issues them instead of
// hiding it behind the next one.  Here the copies that a phase hands on are
// waited for explicitly (wait_tile_loads) by the waves that issued them, so
// the barrier itself only has to order LDS reads: this wave's are drained
// (lgkmcnt) and the "memory" clobber keeps the compiler from moving LDS
// accesses across it.
__device__ __forceinline__ void phase_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <bool SET_M>
__device__ __forceinline__ void pp_vphase(WaveAttn& st, f32x16& s0, f32x16& s1, int k,
                                          int n_unm, int lim_abs, int h2, u32x4 (&pb)[4]) {
  if (k >= n_unm) WaveAttn::mask(s0, s1, k * kKeyTile, lim_abs, h2);
  if (SET_M && k == 0) st.m = WaveAttn::row_max(s0, s1);
  st.probs<false>(s0, s1, k * kKeyTile, lim_abs, h2, pb);
  pin(pb, st.lsum);
}

// M(k+1) with the buffers of parity PAR = k & 1: P.V of tile k from
// v[PAR], then Q.K of tile k+1 from k[1-PAR].
template <int PAR>
__device__ __forceinline__ void pp_mphase(WaveAttn& st, const AttnLds& lds, uint32_t kbt,
                                          uint32_t vbt, const u32x4 (&qb)[8],
                                          const u32x4 (&pb)[4], f32x16& s0, f32x16& s1,
                                          bool has_next) {
  // after the last tile the QK product reads a stale buffer; its result is unused
  (void)has_next;
  st.pv_qk<true>(PAR ? lds.v1 : lds.v0, vbt, pb, PAR ? lds.k0 : lds.k1, kbt, qb, s0, s1);
  pin(s0, s1);
  pin(st.o);
}

// The claim of a workgroup's next q-tile from the tile counter.  One lane
// (kClaimThread, in group B) takes it kClaimLead key tiles before the end of
// the current q-tile: late enough that the tile goes to whichever workgroup
// frees up first (a claim at the start of a long q-tile would hold the next
// one back behind it while other CUs idle), early enough that the counter's
// round trip is hidden behind the last key tiles.
constexpr int kClaimThread = 256, kClaimLead = 2;
struct NextClaim {
  int* ctr;
  int at;     // key tile at which this wave claims; -1: none (wave-uniform)
  int count;  // the count taken (lane kClaimThread), -1 before the claim;
              // used only after the q-tile, so the atomic's return is not
              // waited for in the middle of it
  __device__ __forceinline__ void at_tile(int kk) {
    if (kk == at) {
      if (threadIdx.x == kClaimThread)
        count = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      at = -1;
    }
  }
};

template <bool IS_B, bool SET_M>
__device__ __forceinline__ void pingpong(WaveAttn& st, const TileLoader<4>& ld,
                                         const AttnLds& lds, const uint16_t* kbase,
                                         const uint16_t* vbase, int64_t sp, int kend,
                                         int n_kt, int n_unm, const u32x4 (&qb)[8],
                                         int lim_abs, int h2, NextClaim& nc) {
  uint32_t kbt, vbt;
  st.offsets(kbt, vbt);
  f32x16 s0, s1;
  u32x4 pb[4];
  // phase 0 (K tile 0 is in k0 and visible; K tile 1 and V tile 0 were
  // issued with it by every wave, see load_next_two).  From here on group B,
  // whose even phases are its exponential phases, issues every tile copy;
  // group A only computes.
  if (!IS_B) {
    WaveAttn::qk(lds.k0, kbt, qb, s0, s1);
    pin(s0, s1);
  }
  phase_barrier();
  if (IS_B) {  // phase 1
    WaveAttn::qk(lds.k0, kbt, qb, s0, s1);
    pin(s0, s1);
    wait_tile_loads();
    phase_barrier();
  }
  for (int k = 0; k < n_kt; k += 2) {
#pragma unroll
    for (int par = 0; par < 2; ++par) {
      const int kk = k + par;
      if (par == 1 && kk >= n_kt) break;
      if (!IS_B) {
        pp_vphase<SET_M>(st, s0, s1, kk, n_unm, lim_abs, h2, pb);  // phase 2kk+1
        wait_tile_loads();
        phase_barrier();
        if (par == 0)  // phase 2kk+2
          pp_mphase<0>(st, lds, kbt, vbt, qb, pb, s0, s1, kk + 1 < n_kt);
        else
          pp_mphase<1>(st, lds, kbt, vbt, qb, pb, s0, s1, kk + 1 < n_kt);
        phase_barrier();
      } else {
        nc.at_tile(kk);  // the atomic's return is waited for with the copies
        if (par == 0) pp_loads<1>(ld, lds, kbase, vbase, sp, kend, kk + 1, n_kt);
        else pp_loads<0>(ld, lds, kbase, vbase, sp, kend, kk + 1, n_kt);
        pp_vphase<SET_M>(st, s0, s1, kk, n_unm, lim_abs, h2, pb);  // phase 2kk+2
        phase_barrier();
        if (par == 0) pp_mphase<0>(st, lds, kbt, vbt, qb, pb, s0, s1, kk + 1 < n_kt);
        else pp_mphase<1>(st, lds, kbt, vbt, qb, pb, s0, s1, kk + 1 < n_kt);
        wait_tile_loads();  // phase 2kk+3
        phase_barrier();
      }
    }
  }
  if (!IS_B) {  // phase 2 n_kt + 1: group B's last M phase
    wait_tile_loads();
    phase_barrier();
  }
}

// The cos/sin rows (512 bytes each) of the block's TQ tokens into LDS, for
// blocks of four or more heads per token (their rows are then shared by that
// many lanes, which would otherwise each read them from L2).  Chunk c of row
// r lands at chunk position c ^ (r & 31), so a wave reading one chunk of 32
// rows hits distinct banks: a copy places lane L at 16 L, so lane L fetches
// the chunk that belongs there.  Rows at or past n_tok read as zero.
template <int TQ>
__device__ __forceinline__ void load_cs_rows(const float2* cs, int tok0, int n_tok,
                                             unsigned char* dst, int w, int l) {
  constexpr int NPIECE = TQ / 2;  // 1 KiB copies, two rows each
  static_assert(NPIECE % 8 == 0, "rows per block");
  const int nrec = __builtin_amdgcn_readfirstlane(n_tok * 512);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(cs + (size_t)tok0 * kHalf), 0, nrec, 0x00020000);
#pragma unroll
  for (int i = 0; i < NPIECE / 8; ++i) {
    const int piece = w + 8 * i;
    const int r = 2 * piece + (l >> 5);
    const int c = (l & 31) ^ (r & 31);
    buffer_load_lds16(rs, dst + piece * 1024, (uint32_t)(r * 512 + c * 16));
  }
}

// K tile 1 and V tile 0 (the copies of the ping-pong's phase 0), issued by all
// eight waves before the block's first barrier: two copies per tile and wave,
// so four copies follow K tile 0 in every wave's memory counter.  K tile 1 is
// copied even past kend (as zeros) to keep that count fixed.
__device__ __forceinline__ void load_next_two(const TileLoader<8>& ld, const AttnLds& lds,
                                              const uint16_t* kbase, const uint16_t* vbase,
                                              int64_t sp, int kend) {
  ld.load_k(kbase, sp, kKeyTile, kend, lds.k1);
  ld.load_v(vbase, sp, 0, kend, lds.v0);
}
// Wait for every copy of this wave but the four of load_next_two.
__device__ __forceinline__ void wait_first_tile() {
  __builtin_amdgcn_s_waitcnt(0x0F74);  // vmcnt(4)
}

template <bool SET_M>
__device__ __forceinline__ void attend_pp(WaveAttn& st, const TileLoader<4>& ld,
                                          const AttnLds& lds, const uint16_t* kbase,
                                          const uint16_t* vbase, int64_t sp, int kend,
                                          int n_kt, int n_unm, const u32x4 (&qb)[8],
                                          int lim_abs, int h2, bool is_b, NextClaim& nc) {
  if (is_b) pingpong<true, SET_M>(st, ld, lds, kbase, vbase, sp, kend, n_kt, n_unm, qb, lim_abs, h2, nc);
  else pingpong<false, SET_M>(st, ld, lds, kbase, vbase, sp, kend, n_kt, n_unm, qb, lim_abs, h2, nc);
}

// Work items are q-tiles, numbered heaviest first; when the number of
// (sequence, kv head) pairs is a multiple of 8, items x and x + 8 belong to
// pairs of the same residue mod 8.  One q-tile: TQ tokens x G heads of one
// (sequence, kv head), 256 query rows on 8 waves.
template <int G>
__device__ __forceinline__ void prefill_tile(const PrefillArgs& a, int x, const AttnLds& lds,
                                             unsigned char* lds_cs, NextClaim& nc) {
  constexpr int TQ = 256 / G;            // tokens per workgroup
  constexpr int NPOS = (TQ + 63) / 64;   // positions per lane (each wave reads all)
  constexpr bool CS_LDS = G >= 4;
  const int tid = threadIdx.x, l = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = l & 31, h2 = l >> 5;

  const int n_pairs = a.n_seq * a.n_kv_heads;
  int pair, qt_rev;
  if ((n_pairs & 7) == 0) {
    const int ppx = n_pairs >> 3, slot = x >> 3;
    pair = (slot % ppx) * 8 + (x & 7);
    qt_rev = slot / ppx;
  } else {
    pair = x % n_pairs;
    qt_rev = x / n_pairs;
  }
  const int seq = pair / a.n_kv_heads, g = pair % a.n_kv_heads;
  const int qt = a.n_qtiles - 1 - qt_rev;
  const uint16_t* kbase = a.c.k + (size_t)seq * a.c.sb + (size_t)g * a.c.sh;
  const uint16_t* vbase = a.c.v + (size_t)seq * a.c.sb + (size_t)g * a.c.sh;

  // K tile 0 first, ahead of the positions it would otherwise wait for: its
  // rows are bounded by the capacity only, since a key at or past the block's
  // last position is masked for every query by selection (so whatever such
  // a row holds never reaches a result).  Every return below first drains it.
  TileLoader<8> ld;  // all waves: the first copies, exact-max pass
  ld.init(w, l, a.c.sp);
  ld.load_k(kbase, a.c.sp, 0, a.c.capacity, lds.k0);

  const int s0 = a.cu_seqlens[seq], s1 = a.cu_seqlens[seq + 1];
  if (s0 < 0 || s1 < s0 || s1 > a.total_tokens || s1 - s0 > a.max_seqlen) {
    if (tid == 0) flag_error(a.err, QA_DEVERR_SEQLENS);
    wait_tile_loads();
    return;
  }
  const int tok0 = s0 + qt * TQ;
  const int n_tok = min(TQ, s1 - tok0);
  if (n_tok <= 0) {
    wait_tile_loads();
    return;
  }

  // this lane's query column
  const int r = 32 * w + j;
  const int hl = r / TQ, tl = r % TQ;
  const int h = g * G + hl;
  const bool tok_ok = tl < n_tok;
  const int t = tok0 + tl;

  // Positions of the block's tokens: every wave reads all of them and
  // reduces in registers (no LDS round trip or barrier).  The q-side reads
  // go out together with them.
  int pv[NPOS];
#pragma unroll
  for (int i = 0; i < NPOS; ++i)
    pv[i] = (l + 64 * i < n_tok) ? a.positions[tok0 + l + 64 * i] : -1;
  QPrologue qp;
  if constexpr (CS_LDS) {
    qp.load_qw(a.q + (size_t)t * a.q_tok_stride + (size_t)h * kHeadDim, tok_ok, a.q_norm_w,
               h2);
    load_cs_rows<TQ>(a.cs, tok0, n_tok, lds_cs, w, l);
  } else {
    qp.load(a.q + (size_t)t * a.q_tok_stride + (size_t)h * kHeadDim, tok_ok,
            a.cs + (size_t)(tok_ok ? t : 0) * kHalf, a.q_norm_w, h2);
  }

  const int cap = a.c.capacity;
  int kv_end = 0, pmin = INT_MAX;
#pragma unroll
  for (int i = 0; i < NPOS; ++i) {
    const bool v = pv[i] >= 0 && pv[i] < cap;
    kv_end = max(kv_end, v ? pv[i] + 1 : 0);
    pmin = min(pmin, v ? pv[i] : INT_MAX);
  }
#pragma unroll
  for (int sh = 1; sh < 64; sh <<= 1) {
    kv_end = max(kv_end, __shfl_xor(kv_end, sh));
    pmin = min(pmin, __shfl_xor(pmin, sh));
  }
  // wave-uniform (the tile loader's buffer descriptors must live in SGPRs)
  kv_end = __builtin_amdgcn_readfirstlane(kv_end);
  pmin = __builtin_amdgcn_readfirstlane(pmin);
  int p = -1;
#pragma unroll
  for (int i = 0; i < NPOS; ++i) {
    const int pi = __shfl(pv[i], tl & 63);
    if (tl / 64 == i) p = pi;
  }
  if (!tok_ok) p = -1;
  const bool q_ok = tok_ok && p >= 0 && p < cap;
  if (!q_ok) p = kv_end - 1;  // sees every key; its output is not kept

  uint16_t* orow = a.out + ((size_t)t * a.n_q_heads + h) * kHeadDim;
  if (kv_end == 0) {  // no valid position in the tile
    wait_tile_loads();
    if (tok_ok) {
      const u32x2 z = {0u, 0u};
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4)
          *reinterpret_cast<u32x2*>(orow + 32 * db + 8 * a4 + 4 * h2) = z;
      if (a.lse && h2 == 0) a.lse[(size_t)t * a.n_q_heads + h] = 0.f;
    }
    return;
  }

  const int n_kt = (kv_end + kKeyTile - 1) / kKeyTile;
  // tiles wholly at or below the smallest position need no mask
  const int n_unm = min((pmin + 1) / kKeyTile, n_kt);

  TileLoader<4> ldb;  // group B: the tile copies of the ping-pong
  ldb.init(w & 3, l, a.c.sp);
  load_next_two(ld, lds, kbase, vbase, a.c.sp, kv_end);

  u32x4 qb[8];
  if constexpr (!CS_LDS) qp.compute((float)a.eps, a.qscale, qb);

  WaveAttn st;
  st.init(l);
  wait_first_tile();
  phase_barrier();
  if constexpr (CS_LDS) {  // the cos/sin rows are in LDS now
    qp.cs_from_lds(lds_cs, tl, h2);
    qp.compute((float)a.eps, a.qscale, qb);
  }
  const bool is_b = w >= 4;
  if (w == kClaimThread / 64) nc.at = max(0, n_kt - kClaimLead);
  attend_pp<true>(st, ldb, lds, kbase, vbase, a.c.sp, kv_end, n_kt, n_unm, qb, p, h2, is_b, nc);
  if (__syncthreads_or(st.overflowed())) {
    // a later score far above the first tile's max: redo with the exact one
    st.m = exact_row_max(st, ld, lds, kbase, a.c.sp, 0, kv_end, qb, p, h2);
    st.reset();
    ld.load_k(kbase, a.c.sp, 0, kv_end, lds.k0);
    load_next_two(ld, lds, kbase, vbase, a.c.sp, kv_end);
    wait_first_tile();
    phase_barrier();
    attend_pp<false>(st, ldb, lds, kbase, vbase, a.c.sp, kv_end, n_kt, n_unm, qb, p, h2, is_b, nc);
  }

  const float lt = st.lsum + __shfl_xor(st.lsum, 32);
  const float inv = q_ok ? 1.0f / lt : 0.f;
  if (tok_ok) {
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        u32x2 pr = {0u, 0u};
        if (q_ok) {
          pr[0] = pack_bf16x2(st.o[db][4 * a4] * inv, st.o[db][4 * a4 + 1] * inv);
          pr[1] = pack_bf16x2(st.o[db][4 * a4 + 2] * inv, st.o[db][4 * a4 + 3] * inv);
        }
        *reinterpret_cast<u32x2*>(orow + 32 * db + 8 * a4 + 4 * h2) = pr;
      }
    if (a.lse && h2 == 0)
      a.lse[(size_t)t * a.n_q_heads + h] =
          q_ok ? (st.m + __log2f(lt)) * kLn2 : 0.f;
  }
}

// Persistent grid, one workgroup per CU: workgroup b starts on q-tile b, and
// after that takes the next q-tile of its XCD's share (tiles r, r + 8, ...
// for XCD r = b mod 8, where the hardware deals block b) from that XCD's
// counter in the workspace (zeroed by the K/V prologue of the same call), so
// the heaviest tiles start first, every CU stays busy to the end, and the
// tiles of one (sequence, kv head) pair stay with the L2 that holds its K and
// V.  The next tile is claimed shortly before the current one ends
// (NextClaim), or after it when it had no key tiles to attend; the first
// tiles are not claimed at all, so a workgroup that starts early cannot take
// a second tile while one that starts late finds none.
template <int G>
__global__ __launch_bounds__(512, 1) void prefill_attn_kernel(PrefillArgs a) {
  constexpr int TQ = 256 / G;
  constexpr bool CS_LDS = G >= 4;
  __shared__ __attribute__((aligned(16))) unsigned char lds_k0[kKTileBytes];
  __shared__ __attribute__((aligned(16))) unsigned char lds_k1[kKTileBytes];
  __shared__ __attribute__((aligned(16))) unsigned char lds_v0[kKTileBytes];
  __shared__ __attribute__((aligned(16))) unsigned char lds_v1[kKTileBytes];
  __shared__ __attribute__((aligned(16))) unsigned char lds_cs[CS_LDS ? TQ * 512 : 16];
  __shared__ int s_item;
  const AttnLds lds{lds_k0, lds_k1, lds_v0, lds_v1};
  const int n_items = a.n_seq * a.n_kv_heads * a.n_qtiles;
  const int xcd = blockIdx.x % kPrefillXcds;
  // the XCD's tiles taken by the first round (one per block of the XCD)
  const int first = ((int)gridDim.x - xcd + kPrefillXcds - 1) / kPrefillXcds;
  int* const ctr = a.tile_ctr + xcd;
  int x = blockIdx.x;  // the grid is never wider than the item count
  while (x < n_items) {
    NextClaim nc{ctr, -1, -1};
    prefill_tile<G>(a, x, lds, lds_cs, nc);
    wait_tile_loads();  // no copy into LDS outlives the tile
    __syncthreads();    // nor any LDS read; every wave has read s_item
    if (threadIdx.x == kClaimThread) {
      const int c = nc.count >= 0
                        ? nc.count
                        : __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_item = xcd + kPrefillXcds * (first + c);
    }
    __syncthreads();
    x = s_item;
  }
}

hipError_t launch_prefill(const PrefillArgs& a0, const RopeFreq& f, int group,
                          hipStream_t s, int* n_kernels) {
  PrefillArgs a = a0;
  *n_kernels = 0;
  if (a.total_tokens == 0) return hipSuccess;
  hipLaunchKernelGGL(kv_prologue_kernel, dim3((a.total_tokens + 3) / 4),
                     dim3(256), 0, s, a, f);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  ++*n_kernels;
  const int tq = 256 / group;
  a.n_qtiles = (a.max_seqlen + tq - 1) / tq;
  int dev = 0, n_cu = 0;
  e = hipGetDevice(&dev);
  if (e == hipSuccess)
    e = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const long n_items = (long)a.n_seq * a.n_kv_heads * a.n_qtiles;
  // a wider item count gets a whole number of blocks per XCD, so that every
  // XCD's share of the tiles has workgroups to take it
  const long n_wg = n_items <= n_cu ? n_items : std::max(kPrefillXcds, n_cu / kPrefillXcds * kPrefillXcds);
  const dim3 grid((unsigned)n_wg);
  switch (group) {
    case 1: hipLaunchKernelGGL(prefill_attn_kernel<1>, grid, dim3(512), 0, s, a); break;
    case 2: hipLaunchKernelGGL(prefill_attn_kernel<2>, grid, dim3(512), 0, s, a); break;
    case 4: hipLaunchKernelGGL(prefill_attn_kernel<4>, grid, dim3(512), 0, s, a); break;
    case 8: hipLaunchKernelGGL(prefill_attn_kernel<8>, grid, dim3(512), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  e = hipGetLastError();
  if (e == hipSuccess) ++*n_kernels;
  return e;
}

}  // namespace qa
