// Attention epilogue on gfx950: output projection with the residual add, then
// the post-attention RMSNorm.
//
// "dryft-flash-infer" agent guide, Where the wins are: RMSNorm, rotary and
// the attention epilogue are small and safe to fuse; Numerics: sums may be
// reordered and accumulated in fp32, the bf16 casts stay where the reference
// has them.  Kernel 1 is a bf16 MFMA GEMM, out[T][hidden] = o[T][in] .
// w_o[hidden][in]^T with fp32 sums, whose epilogue rounds each sum to bf16
// (the linear layer's output), adds the residual stream element and rounds
// again (the bf16 residual add), writing the new residual in place.
// Kernel 2 is the hidden-state RMSNorm of rmsnorm.hip on that residual.
//
// GEMM tiling: a workgroup of eight waves owns a 256 x 128 output tile, as
// 4 x 2 waves of 64 x 64 (2 x 2 blocks of v_mfma_f32_32x32x16_bf16, tokens on
// the MFMA row axis, output features on the column axis, both operands read
// with K contiguous: the linear layer's weight is [out][in]).  K advances 64
// at a time through a ring of three LDS stages filled by buffer_load ... lds
// (no register staging): a stage is 1 KiB pieces of 8 rows x 128 B, and each
// 16-byte chunk c of row r sits at chunk position c ^ (r & 7), so the operand
// reads of 32 rows hit distinct banks; a copy lands lane L at byte 16 L of
// its piece, so lane L fetches the chunk that belongs there.  Each step waits
// only for its own stage (the next one stays in flight) and refills the
// stage the previous step used.
//
// Decode-sized batches (at most kEpSmallT tokens) take a second kernel: the
// GEMM grid would be a few tiles wide there, while the work is one streaming
// read of w_o.  A workgroup owns nf <= kEpSmallN output features, nf chosen so
// that the grid covers the CUs (10 for hidden 2560: 256 workgroups, where 16
// would leave 96 CUs without a share of the stream), and its eight waves
// split K into eighths; each lane holds its wave's slice of those weight rows
// in registers (all loads in flight at once), token tiles of 16 run
// v_mfma_f32_16x16x32_bf16 over them (tokens on the row axis, the 16
// features on the column axis), and the eight
// partial sums of an output are added in wave order through LDS, so the
// result does not depend on timing.
#include <algorithm>

#include "attn_tile.h"
#include "qa.h"
#include "qa_device.h"
#include "qa_internal.h"
#include "rmsnorm.h"

namespace qa {

// The streaming kernel's grid aims at this many workgroups (one per CU).
constexpr int kEpSmallCUs = 256;

// LDS byte offset of chunk c of row r in a stage (128-byte rows).
__device__ __forceinline__ uint32_t ep_swz(int row, int chunk) {
  return (uint32_t)(row * 128 + ((chunk ^ (row & 7)) << 4));
}

__device__ __forceinline__ uint16_t f_to_bf(float x) {
  return (uint16_t)(pack_bf16x2(x, 0.f) & 0xffffu);
}

// One K step of the wave's 64 x 64 quarter from the stage (sa, sb).
__device__ __forceinline__ void ep_mma_stage(const unsigned char* sa, const unsigned char* sb,
                                             int wm, int wn, int lr, int h,
                                             f32x16 (&acc)[2][2]) {
#pragma unroll
  for (int ks = 0; ks < kEpBK / 16; ++ks) {
    const int ch = 2 * ks + h;
    u32x4 av[2], bv[2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
      av[i] = *reinterpret_cast<const u32x4*>(sa + ep_swz(wm + 32 * i + lr, ch));
#pragma unroll
    for (int j = 0; j < 2; ++j)
      bv[j] = *reinterpret_cast<const u32x4*>(sb + ep_swz(wn + 32 * j + lr, ch));
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = mfma32x32x16(av[i], bv[j], acc[i][j]);
  }
}

// The GEMM's LDS stages, selected by compile-time index so that the compiler
// sees which array each read and each copy touches (a copy in flight into
// one stage then does not hold up reads of another).
struct EpStages {
  unsigned char *a0, *a1, *a2, *b0, *b1, *b2;
};
template <int S>
__device__ __forceinline__ unsigned char* ep_a(const EpStages& t) {
  if constexpr (S == 0) return t.a0;
  else if constexpr (S == 1) return t.a1;
  else return t.a2;
}
template <int S>
__device__ __forceinline__ unsigned char* ep_b(const EpStages& t) {
  if constexpr (S == 0) return t.b0;
  else if constexpr (S == 1) return t.b1;
  else return t.b2;
}

// Copies of one K step: A has kEpBM / 8 pieces of 1 KiB per stage, B
// kEpBN / 8; wave w takes pieces w, w + 8, ...
struct EpCopies {
  static constexpr int NA = kEpBM / 64, NB = kEpBN / 64;  // pieces per wave
  __amdgpu_buffer_rsrc_t ra, rb;
  uint32_t aoff[NA], boff[NB];
  int w;
  __device__ __forceinline__ void load(int kt, unsigned char* da, unsigned char* db) const {
    const uint32_t ko = (uint32_t)kt * (kEpBK * 2);
#pragma unroll
    for (int i = 0; i < NA; ++i) buffer_load_lds16(ra, da + (w + 8 * i) * 1024, aoff[i] + ko);
#pragma unroll
    for (int i = 0; i < NB; ++i) buffer_load_lds16(rb, db + (w + 8 * i) * 1024, boff[i] + ko);
  }
};

// Step kt (stage S = kt % 3): wait for stage S (only stage kt+1's copies stay
// in flight), barrier (every wave's pieces landed; every read of the stage
// about to be refilled, used at step kt-1, done), refill that stage with
// kt+2, then the MFMAs of stage S.  The refill is issued even past the last
// step (it reads finite data or zeros into a stage nobody reads again), so
// that the count of copies in flight, and the compiler's view of which stage
// they write, never depend on a branch.
template <int S>
__device__ __forceinline__ void ep_step(const EpStages& st, const EpCopies& cp, int kt,
                                        int wm, int wn, int lr, int h, f32x16 (&acc)[2][2]) {
  wait_vmcnt<EpCopies::NA + EpCopies::NB>();
  lds_barrier();
  cp.load(kt + 2, ep_a<(S + 2) % 3>(st), ep_b<(S + 2) % 3>(st));
  ep_mma_stage(ep_a<S>(st), ep_b<S>(st), wm, wn, lr, h, acc);
}

__global__ __launch_bounds__(512) void epilogue_gemm_kernel(EpilogueArgs a) {
  constexpr int kAB = kEpBM * 128, kBB = kEpBN * 128;  // stage bytes
  __shared__ __attribute__((aligned(16))) unsigned char sA0[kAB];
  __shared__ __attribute__((aligned(16))) unsigned char sA1[kAB];
  __shared__ __attribute__((aligned(16))) unsigned char sA2[kAB];
  __shared__ __attribute__((aligned(16))) unsigned char sB0[kBB];
  __shared__ __attribute__((aligned(16))) unsigned char sB1[kBB];
  __shared__ __attribute__((aligned(16))) unsigned char sB2[kBB];
  const EpStages st{sA0, sA1, sA2, sB0, sB1, sB2};
  const int tid = threadIdx.x, l = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Workgroups are dealt to the 8 XCDs round-robin by id: XCD x takes the
  // token tiles x, x + 8, ... with the feature tiles varying fastest, so the
  // n_nt workgroups that read one token tile of o share one L2.  Ids past the
  // last token tile (the grid is rounded up to 8 of them) exit.
  const int n_nt = a.hidden / kEpBN;
  const int xcd = blockIdx.x & 7, li = blockIdx.x >> 3;
  const int m0 = (xcd + 8 * (li / n_nt)) * kEpBM, n0 = (li % n_nt) * kEpBN;
  if (m0 >= a.n_tokens) return;  // (workgroup-uniform, before any barrier)
  const int wm = (w >> 1) * 64, wn = (w & 1) * 64;  // this wave's quarter

  // Token rows at or past the last read as zeros (the buffer's range ends
  // there).  In a piece, lane L lands at byte 16 L: row 8p + L/8, position
  // L%8, which holds logical chunk (L%8) ^ (L/8).
  EpCopies cp;
  cp.w = w;
  const int prow = l >> 3, pchunk = (l & 7) ^ (l >> 3);
  const uint32_t os2 = (uint32_t)a.o_stride * 2u, is2 = (uint32_t)a.in_dim * 2u;
  const int rows_left = min(kEpBM, a.n_tokens - m0);
  cp.ra = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.o + (size_t)m0 * a.o_stride), 0,
      __builtin_amdgcn_readfirstlane(rows_left * (int)os2), 0x00020000);
  cp.rb = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.w + (size_t)n0 * a.in_dim), 0,
      __builtin_amdgcn_readfirstlane(kEpBN * (int)is2), 0x00020000);
#pragma unroll
  for (int i = 0; i < EpCopies::NA; ++i)
    cp.aoff[i] = (uint32_t)(8 * (w + 8 * i) + prow) * os2 + 16u * pchunk;
#pragma unroll
  for (int i = 0; i < EpCopies::NB; ++i)
    cp.boff[i] = (uint32_t)(8 * (w + 8 * i) + prow) * is2 + 16u * pchunk;

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  const int lr = l & 31, h = l >> 5;
  const int nk = a.in_dim / kEpBK;
  cp.load(0, sA0, sB0);
  cp.load(1, sA1, sB1);
  int kt = 0;
  for (; kt + 3 <= nk; kt += 3) {
    ep_step<0>(st, cp, kt, wm, wn, lr, h, acc);
    ep_step<1>(st, cp, kt + 1, wm, wn, lr, h, acc);
    ep_step<2>(st, cp, kt + 2, wm, wn, lr, h, acc);
  }
  if (kt < nk) ep_step<0>(st, cp, kt, wm, wn, lr, h, acc);
  if (kt + 1 < nk) ep_step<1>(st, cp, kt + 1, wm, wn, lr, h, acc);
  wait_vmcnt<0>();  // no copy into LDS outlives the workgroup

  // epilogue: h = bf16(sum), r = bf16(h + residual), written over the residual
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = n0 + wn + 32 * j + lr;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm + 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);
        if (row < a.n_tokens) {
          uint16_t* rp = a.res + (size_t)row * a.hidden + col;
          const float hv = bf_to_f(f_to_bf(acc[i][j][r]));
          *rp = f_to_bf(hv + bf_to_f(*rp));
        }
      }
    }
}

// nf: output features per workgroup (1 .. kEpSmallN); MFMA columns from nf
// on, and features past the hidden size in the last workgroup, repeat a
// valid weight row and are never stored.
template <int KS>
__global__ __launch_bounds__(512) void epilogue_small_kernel(EpilogueArgs a, int nf) {
  static_assert(kEpSmallN == 16, "one feature per MFMA column");
  __shared__ float part[8][16][kEpSmallN + 1];
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int n0 = blockIdx.x * nf;
  const int kw = w * (32 * KS);  // this wave's K range: kw .. kw + 32 KS - 1
  const int kq = 8 * (l >> 4);   // the lane's 8 k values within a 32-wide step
  // B operand of step s: W[n0 + (l & 15)][kw + 32 s + kq .. +7]
  u32x4 wb[KS];
  const int wf = min(n0 + min(l & 15, nf - 1), a.hidden - 1);
  const uint16_t* wrow = a.w + (size_t)wf * a.in_dim + kw + kq;
#pragma unroll
  for (int s = 0; s < KS; ++s) wb[s] = ld16(wrow + 32 * s);
  // the residual element each of the first 256 threads adds to, read now so
  // that its latency overlaps the weight stream (the next tile's is read
  // after this tile's store)
  const int tr = tid / nf, f = tid - tr * nf;
  const bool fout = tid < 16 * nf && n0 + f < a.hidden;  // (token row, feature) of this thread
  uint16_t* rp = a.res + (size_t)min(tr, a.n_tokens - 1) * a.hidden + min(n0 + f, a.hidden - 1);
  uint16_t rv = fout ? *rp : (uint16_t)0;
  for (int t0 = 0; t0 < a.n_tokens; t0 += 16) {
    const int tt = min(t0 + (l & 15), a.n_tokens - 1);  // rows past the last repeat it
    const uint16_t* orow = a.o + (size_t)tt * a.o_stride + kw + kq;
    u32x4 ob[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) ob[s] = ld16(orow + 32 * s);
    // all KS loads in flight before the first MFMA: left alone, the compiler
    // pipelines them two deep, and each MFMA then waits a round trip to L2
    __builtin_amdgcn_sched_barrier(0);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) acc = mfma16x16x32(ob[s], wb[s], acc);
    // D: lane l holds tokens t0 + 4 (l >> 4) + r of feature column l & 15
#pragma unroll
    for (int r = 0; r < 4; ++r) part[w][4 * (l >> 4) + r][l & 15] = acc[r];
    __syncthreads();
    if (fout) {
      const int tok = t0 + tr;
      float sum = part[0][tr][f];
#pragma unroll
      for (int v = 1; v < 8; ++v) sum += part[v][tr][f];
      if (tok < a.n_tokens) {
        const float h = bf_to_f(f_to_bf(sum));
        *rp = f_to_bf(h + bf_to_f(rv));
      }
      if (tok + 16 < a.n_tokens) {
        rp += (size_t)16 * a.hidden;
        rv = *rp;
      }
    }
    __syncthreads();  // part is rewritten by the next token tile
  }
}

hipError_t launch_attn_epilogue(const EpilogueArgs& a, const NormArgs& n, hipStream_t s,
                                int* n_kernels) {
  *n_kernels = 0;
  if (a.n_tokens == 0) return hipSuccess;
  const int ks = a.in_dim / 256;  // K steps of 32 per wave on the small path
  const bool small = a.n_tokens <= kEpSmallT && a.in_dim % 256 == 0 &&
                     (ks == 2 || ks == 4 || ks == 8 || ks == 16 || ks == 32);
  if (small) {
    const int nf = std::min(kEpSmallN, std::max(1, (a.hidden + kEpSmallCUs - 1) / kEpSmallCUs));
    const dim3 grid((a.hidden + nf - 1) / nf);
    switch (ks) {
      case 2: hipLaunchKernelGGL(epilogue_small_kernel<2>, grid, dim3(512), 0, s, a, nf); break;
      case 4: hipLaunchKernelGGL(epilogue_small_kernel<4>, grid, dim3(512), 0, s, a, nf); break;
      case 8: hipLaunchKernelGGL(epilogue_small_kernel<8>, grid, dim3(512), 0, s, a, nf); break;
      case 16: hipLaunchKernelGGL(epilogue_small_kernel<16>, grid, dim3(512), 0, s, a, nf); break;
      default: hipLaunchKernelGGL(epilogue_small_kernel<32>, grid, dim3(512), 0, s, a, nf); break;
    }
  } else {
    const int n_mt = (a.n_tokens + kEpBM - 1) / kEpBM;
    const dim3 grid((unsigned)((a.hidden / kEpBN) * 8 * ((n_mt + 7) / 8)));
    hipLaunchKernelGGL(epilogue_gemm_kernel, grid, dim3(512), 0, s, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  *n_kernels = 1;
  e = launch_rmsnorm_hidden(n, s);
  if (e == hipSuccess) *n_kernels = 2;
  return e;
}

}  // namespace qa
