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
// GEMM tiling: a workgroup of four waves owns a 128 x 128 output tile; K
// advances 64 at a time through two LDS stages (register staged: the next
// stage's global loads are issued before the current stage's MFMAs), each
// 16-byte chunk c of a 128-byte LDS row r stored at chunk c ^ (r & 7) so the
// operand reads of 32 rows hit distinct banks.  Wave (i, j) computes the
// 64 x 64 quarter (i, j) as 2 x 2 blocks of v_mfma_f32_32x32x16_bf16, tokens
// on the MFMA row axis and output features on the column axis, both operands
// read with K contiguous (the linear layer's weight is [out][in]).
//
// Decode-sized batches (at most kEpSmallT tokens) take a second kernel: the
// GEMM grid would be a few tiles wide there, while the work is one streaming
// read of w_o.  A workgroup owns kEpSmallN output features and its eight waves
// split K into eighths; each lane holds its wave's slice of those weight rows
// in registers (all loads in flight at once), token tiles of 16 run
// v_mfma_f32_16x16x32_bf16 over them (tokens on the row axis, the 16
// features on the column axis), and the eight
// partial sums of an output are added in wave order through LDS, so the
// result does not depend on timing.
#include "qa.h"
#include "qa_device.h"
#include "qa_internal.h"
#include "rmsnorm.h"

namespace qa {

__device__ __forceinline__ uint32_t ep_swz(int row, int chunk) {
  return (uint32_t)(row * 128 + ((chunk ^ (row & 7)) << 4));
}

__device__ __forceinline__ uint16_t f_to_bf(float x) {
  return (uint16_t)(pack_bf16x2(x, 0.f) & 0xffffu);
}

__global__ __launch_bounds__(256) void epilogue_gemm_kernel(EpilogueArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char sA[2][kEpBM * 128];
  __shared__ __attribute__((aligned(16))) unsigned char sB[2][kEpBN * 128];
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  // Workgroups are dealt to the 8 XCDs round-robin by id: XCD x takes the
  // token tiles x, x + 8, ... with the feature tiles varying fastest, so the
  // n_nt workgroups that read one token tile of o share one L2.  Ids past the
  // last token tile (the grid is rounded up to 8 of them) exit.
  const int n_nt = a.hidden / kEpBN;
  const int xcd = blockIdx.x & 7, li = blockIdx.x >> 3;
  const int m0 = (xcd + 8 * (li / n_nt)) * kEpBM, n0 = (li % n_nt) * kEpBN;
  if (m0 >= a.n_tokens) return;  // (workgroup-uniform, before any barrier)
  const int wm = (w >> 1) * 64, wn = (w & 1) * 64;

  // 16-byte chunks tid + 256 j (j < 4) of each 128 x 64 stage: row id >> 3,
  // chunk id & 7; token rows past the last are read from the last one (their
  // results are not stored)
  u32x4 ra[4], rb[4];
  auto gload = [&](int kt) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int id = tid + 256 * j, row = id >> 3, c = id & 7;
      const int m = min(m0 + row, a.n_tokens - 1);
      ra[j] = ld16(a.o + (size_t)m * a.o_stride + kt * kEpBK + 8 * c);
      rb[j] = ld16(a.w + (size_t)(n0 + row) * a.in_dim + kt * kEpBK + 8 * c);
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int id = tid + 256 * j, row = id >> 3, c = id & 7;
      st16(sA[buf] + ep_swz(row, c), ra[j]);
      st16(sB[buf] + ep_swz(row, c), rb[j]);
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk = a.in_dim / kEpBK;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
#pragma unroll
    for (int ks = 0; ks < kEpBK / 16; ++ks) {
      const int ch = 2 * ks + (l >> 5);
      u32x4 av[2], bv[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        av[i] = *reinterpret_cast<const u32x4*>(sA[cur] + ep_swz(wm + 32 * i + (l & 31), ch));
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bv[j] = *reinterpret_cast<const u32x4*>(sB[cur] + ep_swz(wn + 32 * j + (l & 31), ch));
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32x32x16(av[i], bv[j], acc[i][j]);
    }
    if (kt + 1 < nk) lstore(cur ^ 1);
    __syncthreads();
  }

  // epilogue: h = bf16(sum), r = bf16(h + residual), written over the residual
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = n0 + wn + 32 * j + (l & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm + 32 * i + 8 * (r >> 2) + 4 * (l >> 5) + (r & 3);
        if (row < a.n_tokens) {
          uint16_t* rp = a.res + (size_t)row * a.hidden + col;
          const float h = bf_to_f(f_to_bf(acc[i][j][r]));
          *rp = f_to_bf(h + bf_to_f(*rp));
        }
      }
    }
}

template <int KS>
__global__ __launch_bounds__(512) void epilogue_small_kernel(EpilogueArgs a) {
  static_assert(kEpSmallN == 16, "one feature per MFMA column");
  __shared__ float part[8][16][kEpSmallN + 1];
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int n0 = blockIdx.x * kEpSmallN;
  const int kw = w * (32 * KS);  // this wave's K range: kw .. kw + 32 KS - 1
  const int kq = 8 * (l >> 4);   // the lane's 8 k values within a 32-wide step
  // B operand of step s: W[n0 + (l & 15)][kw + 32 s + kq .. +7]
  u32x4 wb[KS];
  const uint16_t* wrow = a.w + (size_t)(n0 + (l & 15)) * a.in_dim + kw + kq;
#pragma unroll
  for (int s = 0; s < KS; ++s) wb[s] = ld16(wrow + 32 * s);
  // the residual element each of the first 256 threads adds to, read now so
  // that its latency overlaps the weight stream (the next tile's is read
  // after this tile's store)
  const int tr = tid / kEpSmallN, f = tid % kEpSmallN;
  uint16_t* rp = a.res + (size_t)min(tr, a.n_tokens - 1) * a.hidden + n0 + f;
  uint16_t rv = tid < 16 * kEpSmallN ? *rp : (uint16_t)0;
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
    if (tid < 16 * kEpSmallN) {
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
    const dim3 grid(a.hidden / kEpSmallN);
    switch (ks) {
      case 2: hipLaunchKernelGGL(epilogue_small_kernel<2>, grid, dim3(512), 0, s, a); break;
      case 4: hipLaunchKernelGGL(epilogue_small_kernel<4>, grid, dim3(512), 0, s, a); break;
      case 8: hipLaunchKernelGGL(epilogue_small_kernel<8>, grid, dim3(512), 0, s, a); break;
      case 16: hipLaunchKernelGGL(epilogue_small_kernel<16>, grid, dim3(512), 0, s, a); break;
      default: hipLaunchKernelGGL(epilogue_small_kernel<32>, grid, dim3(512), 0, s, a); break;
    }
  } else {
    const int n_mt = (a.n_tokens + kEpBM - 1) / kEpBM;
    const dim3 grid((unsigned)((a.hidden / kEpBN) * 8 * ((n_mt + 7) / 8)));
    hipLaunchKernelGGL(epilogue_gemm_kernel, grid, dim3(256), 0, s, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  *n_kernels = 1;
  e = launch_rmsnorm_hidden(n, s);
  if (e == hipSuccess) *n_kernels = 2;
  return e;
}

}  // namespace qa
