// vs_moba.hip — the MoBA block gate (an alternative index estimator) and the
// per-query-block summaries of a per-row block selection.
//
// The MTraining paper note (appendix, baseline settings, item 1) describes
// MoBA: the keys are cut into blocks of fixed size, an MoE-style gate picks
// for every query the top-k blocks, always including the query's own block
// (block 4096, top-12).  Steps:
//   * kbar_J = the mean of key block J's keys (vs_moba_means_kernel);
//   * gate score of block J for query n: q_n . kbar_J, for the blocks J
//     before n's own block;
//   * picked: the own block and the k - 1 highest-scoring earlier blocks
//     (ties to the lowest J), one 32-bit word per row (vs_moba_select_kernel).
// The attention kernels read the words in place of the Vertical-Slash
// lists; the key-major backward also reads, per (batch, Q head, 64-row query
// block), the OR of its rows' words (vs_moba_union_kernel).
#include "vs_attn_common.h"
#include "vs_moba_params.h"
#include "vs_trace.h"

namespace vs {


// One workgroup per (batch, KV head, key block): the mean of its keys.
// Thread t reads 8 channels (c8 = t % (D / 8), one 16-byte load per row) of
// every RG-th row starting at t / (D / 8); the RG partial sums of a channel
// are then added in a fixed order, so the means (and the picks) are the same
// in every run.
template <int D>
__global__ __launch_bounds__(512) void vs_moba_means_kernel(MobaParams p) {
  constexpr int CH = D / 8;        // 16-byte chunks per row
  constexpr int RG = 512 / CH;     // row groups
  __shared__ float part[RG][D];
  const int J = blockIdx.x % p.nB;
  const int bk = blockIdx.x / p.nB;  // b * h_kv + kvh
  const int b = bk / p.h_kv, kvh = bk % p.h_kv;
  const int c8 = threadIdx.x % CH, g = threadIdx.x / CH;
  const int r0 = J * p.blk, r1 = min(r0 + p.blk, p.n);
  const __bf16* kb = p.k + p.sk.at(b, 0, kvh) + 8 * c8;
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  for (int r = r0 + g; r < r1; r += RG) {
    const bf16x8 v = *reinterpret_cast<const bf16x8*>(kb + (size_t)r * p.sk.t);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += (float)v[e];
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) part[g][8 * c8 + e] = acc[e];
  __syncthreads();
  if (threadIdx.x < D) {
    float s = 0.f;
    for (int u = 0; u < RG; ++u) s += part[u][threadIdx.x];
    p.kbar[((size_t)bk * p.nB + J) * D + threadIdx.x] = s / (float)(r1 - r0);
  }
}

// One thread per query row, 256 rows per workgroup (one own block: the
// block size is a multiple of 256): gate scores against the earlier blocks'
// means (kept in LDS, read as broadcasts), then each earlier block's rank
// among them; the k - 1 best and the own block form the row's word.
template <int D>
__global__ __launch_bounds__(256) void vs_moba_select_kernel(MobaParams p) {
  __shared__ float kb[32][D];
  const int rows_per_head = (p.n + 255) / 256;
  const int bh = blockIdx.x / rows_per_head;
  const int r0 = (blockIdx.x % rows_per_head) * 256;
  const int b = bh / p.h_q, h = bh % p.h_q;
  const int kvh = h * p.h_kv / p.h_q;
  const int own = r0 / p.blk;  // every row of the workgroup lies in this block
  for (int e = threadIdx.x; e < own * D; e += 256)
    kb[e / D][e % D] = p.kbar[((size_t)(b * p.h_kv + kvh) * p.nB) * D + e];
  __syncthreads();
  const int row = r0 + threadIdx.x;
  if (row >= p.n) return;
  const __bf16* qr = p.q + p.sq.at(b, row, h);
  float s[32];
#pragma unroll
  for (int J = 0; J < 32; ++J) s[J] = 0.f;
  for (int c = 0; c < D; c += 8) {
    const bf16x8 qv = *reinterpret_cast<const bf16x8*>(qr + c);
    float qf[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) qf[e] = (float)qv[e];
#pragma unroll
    for (int J = 0; J < 32; ++J) {
      if (J < own) {
#pragma unroll
        for (int e = 0; e < 8; ++e) s[J] = __builtin_fmaf(qf[e], kb[J][c + e], s[J]);
      }
    }
  }
  // rank of J among the earlier blocks: higher scores first, ties to the lower index
  uint32_t word = 1u << own;
#pragma unroll
  for (int J = 0; J < 32; ++J) {
    if (J < own) {
      int rank = 0;
#pragma unroll
      for (int I = 0; I < 32; ++I)
        if (I < own && (s[I] > s[J] || (s[I] == s[J] && I < J))) ++rank;
      if (rank < p.topk - 1) word |= 1u << J;
    }
  }
  const size_t ri = (size_t)bh * p.n + row;
  p.rmask[ri] = word;
  if (p.scores) {
#pragma unroll
    for (int J = 0; J < 32; ++J)
      if (J < p.nB) p.scores[ri * p.nB + J] = s[J];
  }
}

hipError_t launch_moba(const MobaParams& p, hipStream_t st) {
  const dim3 gm((unsigned)(p.batch * p.h_kv * p.nB));
  const dim3 gs((unsigned)(p.batch * p.h_q * ((p.n + 255) / 256)));
  if (gs.x == 0) return hipSuccess;
  if (p.d == 128) {
    VS_TRACED(st, "vs_moba_means", hipLaunchKernelGGL((vs_moba_means_kernel<128>), gm, dim3(512), 0, st, p));
    VS_TRACED(st, "vs_moba_select", hipLaunchKernelGGL((vs_moba_select_kernel<128>), gs, dim3(256), 0, st, p));
  } else {
    VS_TRACED(st, "vs_moba_means", hipLaunchKernelGGL((vs_moba_means_kernel<64>), gm, dim3(512), 0, st, p));
    VS_TRACED(st, "vs_moba_select", hipLaunchKernelGGL((vs_moba_select_kernel<64>), gs, dim3(256), 0, st, p));
  }
  return hipGetLastError();
}

// The OR of the 64 rows' words of every (batch, Q head, query block): the
// blocks some row of the query block picked.
__global__ __launch_bounds__(256) void vs_moba_union_kernel(const uint32_t* rmask, uint32_t* out, int tiles) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= tiles) return;
  const uint32_t* w = rmask + (size_t)t * kBlock;
  uint32_t u = 0u;
  for (int r = 0; r < kBlock; ++r) u |= w[r];
  out[t] = u;
}

hipError_t launch_moba_union(const uint32_t* rmask, uint32_t* out, int tiles, hipStream_t st) {
  if (tiles <= 0) return hipSuccess;
  VS_TRACED(st, "vs_moba_union", hipLaunchKernelGGL(vs_moba_union_kernel, dim3((unsigned)((tiles + 255) / 256)),
                                                    dim3(256), 0, st, rmask, out, tiles));
  return hipGetLastError();
}

}  // namespace vs
