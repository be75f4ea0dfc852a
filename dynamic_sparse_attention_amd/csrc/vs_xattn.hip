// vs_xattn.hip — XAttention block estimation (an alternative index estimator).
//
// The MTraining paper note (appendix, baseline settings, item 2) describes
// XAttention: square blocks of the attention matrix are scored by sums along
// their anti-diagonals taken at a stride, and only high-scoring blocks are
// kept (block 128, stride 16, threshold 0.9).  Steps:
//   * cells of S x S (S = 16) are sampled along their anti-diagonal:
//     z[A, C] = (1/S) sum_u scale * q[S A + u] . k[S C + S - 1 - u], causal at
//     cell level (C <= A);
//   * each cell row is normalised by a softmax over its cells;
//   * a block (I, J) of 128 x 128 scores the sum of its cells' probabilities;
//   * each query block keeps the fewest key blocks, highest first (ties to
//     the lowest index), holding the threshold's share of its total.
// The selection is written as a bitmap per (batch, Q head, query block),
// which the attention kernels read in place of the Vertical-Slash lists.
//
// gfx950 design.  vs_xa_cells_kernel: one workgroup (4 waves) per 32 cell
// rows of one (batch, Q head); the cell logits are a contraction over
// S * d = 2048 (16 sample offsets u x d channels), so wave w keeps the Q side
// of offsets u in [4w, 4w + 4) in registers (bf16 B operands) and multiplies
// it with the K rows of the same offsets of each 32-cell column tile
// (v_mfma_f32_32x32x16_bf16, A operand straight from global memory); the four
// partial tiles add up through LDS.  Per cell row and key block (8 cells) it
// stores the log-sum-exp of the block's cells (log2 domain), and per cell row
// the log-sum-exp of the whole row.  vs_xa_select_kernel: one workgroup per
// (batch, Q head, query block) forms the block scores
// s[I, J] = sum over the block's cell rows of 2^(lse[A, J] - lse[A]), takes
// integer masses rint(s * 2^50) (exact and the same in every run), sorts the
// (mass, index) keys with a bitonic sort in LDS and keeps the shortest prefix
// whose mass reaches ceil(rint(t * 2^24) * total / 2^24).
#include "vs_attn_common.h"
#include "vs_trace.h"
#include "vs_xattn_params.h"

namespace vs {

constexpr int kXaStride = 16;      // S
constexpr int kXaBlock = 128;      // block side (tokens)
constexpr int kXaCpb = kXaBlock / kXaStride;  // cells per block side: 8
constexpr int kXaTile = 32;        // cell rows / columns per tile

template <int D>
__global__ __launch_bounds__(256) void vs_xa_cells_kernel(XaParams p) {
  typedef Mfma<__bf16> MF;
  typedef MF::frag frag;
  constexpr int KPL = MF::KPL, KC = 2 * KPL, NCD = D / KC;
  constexpr int UW = kXaStride / 4;  // sample offsets per wave
  __shared__ float red[4][kXaTile][kXaTile + 1];  // [wave][cell col][cell row]
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, hl = lane >> 5, l32 = lane & 31;
  const int n_rt = (p.nC + kXaTile - 1) / kXaTile;
  // heaviest row tiles (most cell columns) first
  const int rt = n_rt - 1 - (int)(blockIdx.x % n_rt);
  const int bh = blockIdx.x / n_rt;
  const int b = bh / p.h_q, h = bh % p.h_q;
  const int kvh = h * p.h_kv / p.h_q;
  const int A0 = rt * kXaTile;
  const __bf16* qb = p.q + p.sq.at(b, 0, h);
  const __bf16* kb = p.k + p.sk.at(b, 0, kvh);

  // Q side (B operand of z^T = K' Q'^T): cell row A0 + l32, offsets u of this wave.
  frag qf[UW][NCD];
  {
    const int A = min(A0 + l32, p.nC - 1);
#pragma unroll
    for (int ui = 0; ui < UW; ++ui) {
      const __bf16* qr = qb + (size_t)(kXaStride * A + UW * wave + ui) * p.sq.t + hl * KPL;
#pragma unroll
      for (int c = 0; c < NCD; ++c) qf[ui][c] = load_frag<__bf16>(qr + c * KC);
    }
  }
  // Reduction role: thread t < 128 owns cell row A0 + t / 4 and key block
  // (of this tile) t % 4, i.e. 8 cell columns.
  const int ra = tid >> 2;
  const int rj = tid & 3;
  float m_row = -INFINITY, l_row = 0.f;  // running log2-domain state of the row
  float* out_lse = p.cell_lse + ((size_t)bh * p.nC + (A0 + ra)) * p.nI;

  for (int ct = 0; ct <= rt; ++ct) {
    const int C0 = ct * kXaTile;
    // A operand: key rows S * (C0 + slot) + S - 1 - u of this wave's offsets;
    // accumulator register i then holds cell column C0 + c_row(i, hl).
    f32x16 acc = f32x16{0};
    const int Cl = min(C0 + l32, p.nC - 1);
#pragma unroll
    for (int ui = 0; ui < UW; ++ui) {
      const int u = UW * wave + ui;
      const __bf16* kr = kb + (size_t)(kXaStride * Cl + kXaStride - 1 - u) * p.sk.t + hl * KPL;
      frag kf[NCD];
#pragma unroll
      for (int c = 0; c < NCD; ++c) kf[c] = load_frag<__bf16>(kr + c * KC);
#pragma unroll
      for (int c = 0; c < NCD; ++c) acc = MF::mma(kf[c], qf[ui][c], acc);
    }
    // acc[i] = partial z of cell column C0 + c_row(i, hl), cell row A0 + l32
#pragma unroll
    for (int i = 0; i < 16; ++i) red[wave][c_row(i, hl)][l32] = acc[i];
    __syncthreads();
    if (tid < 128) {
      const int A = A0 + ra;
      float z[kXaCpb];
      float mx = -INFINITY;
#pragma unroll
      for (int e = 0; e < kXaCpb; ++e) {
        const int cc = kXaCpb * rj + e;
        const int C = C0 + cc;
        const float v = red[0][cc][ra] + red[1][cc][ra] + red[2][cc][ra] + red[3][cc][ra];
        z[e] = (C <= A && C < p.nC) ? v * (p.sl2 / kXaStride) : -INFINITY;
        mx = fmaxf(mx, z[e]);
      }
      float sum = 0.f;
      const float mu = mx == -INFINITY ? 0.f : mx;
#pragma unroll
      for (int e = 0; e < kXaCpb; ++e) sum += fast_exp2(z[e] - mu);
      const float lse_j = sum > 0.f ? mu + __log2f(sum) : -INFINITY;
      const int J = (C0 / kXaCpb) + rj;
      if (A < p.nC && J < p.nI) out_lse[J] = lse_j;
      // row state over the four key blocks of the tile (adjacent lanes)
      float tmax = lse_j;
      tmax = fmaxf(tmax, __shfl_xor(tmax, 1, 64));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 2, 64));
      const float mn = fmaxf(m_row, tmax);
      const float mnu = mn == -INFINITY ? 0.f : mn;
      float add = lse_j == -INFINITY ? 0.f : fast_exp2(lse_j - mnu);
      add += __shfl_xor(add, 1, 64);
      add += __shfl_xor(add, 2, 64);
      l_row = l_row * (m_row == -INFINITY ? 0.f : fast_exp2(m_row - mnu)) + add;
      m_row = mn;
    }
    __syncthreads();
  }
  if (tid < 128 && rj == 0 && A0 + ra < p.nC)
    p.row_lse[(size_t)bh * p.nC + A0 + ra] = l_row > 0.f ? m_row + __log2f(l_row) : -INFINITY;
}

// Bitonic sort of NS 64-bit keys in LDS, descending, by 256 threads.
template <int NS>
__device__ __forceinline__ void bitonic_desc(unsigned long long* key) {
  for (int size = 2; size <= NS; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int t = threadIdx.x; t < NS / 2; t += 256) {
        const int lo = 2 * t - (t & (stride - 1));
        const int hi = lo + stride;
        const bool desc = ((lo & size) == 0);
        const unsigned long long a = key[lo], c = key[hi];
        if ((a < c) == desc) {
          key[lo] = c;
          key[hi] = a;
        }
      }
      __syncthreads();
    }
  }
}

constexpr int kXaMaxBlocks = 1024;  // query blocks per segment the selection sorts (n <= 131072)

__global__ __launch_bounds__(256) void vs_xa_select_kernel(XaParams p) {
  __shared__ unsigned long long key[kXaMaxBlocks];
  __shared__ unsigned long long wsum[4];
  __shared__ uint32_t row_bits[kXaMaxBlocks / 32];
  __shared__ int s_k;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int I = blockIdx.x % p.nI;
  const int bh = blockIdx.x / p.nI;
  const int nJ = I + 1;
  const int a_lo = I * kXaCpb, a_hi = min(a_lo + kXaCpb, p.nC);
  // block scores and their integer masses (exact multiples of 2^-50; s <= 8)
  unsigned long long tot = 0;
  for (int J = tid; J < kXaMaxBlocks; J += 256) {  // every key: past nJ, mass 0 behind the real ones
    unsigned long long w = 0;
    if (J < nJ) {
      float s = 0.f;
      for (int A = a_lo; A < a_hi; ++A) {
        const float cl = p.cell_lse[((size_t)bh * p.nC + A) * p.nI + J];
        const float rl = p.row_lse[(size_t)bh * p.nC + A];
        if (cl != -INFINITY) s += fast_exp2(cl - rl);
      }
      if (p.scores) p.scores[((size_t)bh * p.nI + I) * p.nI + J] = s;
      w = (unsigned long long)rint((double)s * 1125899906842624.0);  // 2^50
    }
    tot += w;
    // (mass, lowest index first): sorted descending by mass, then by 1023 - J
    key[J] = (w << 10) | (unsigned long long)(kXaMaxBlocks - 1 - J);
  }
  for (int o = 32; o > 0; o >>= 1) tot += __shfl_xor(tot, o, 64);
  if (lane == 0) wsum[wave] = tot;
  for (int w = tid; w < kXaMaxBlocks / 32; w += 256) row_bits[w] = 0u;
  __syncthreads();
  tot = wsum[0] + wsum[1] + wsum[2] + wsum[3];
  bitonic_desc<kXaMaxBlocks>(key);
  // target = ceil(rint(t * 2^24) * total / 2^24), t clamped to [0, 1]
  float t = p.threshold;
  t = (t > 0.f) ? fminf(t, 1.f) : 0.f;
  const unsigned long long tq = (unsigned long long)rint((double)t * 16777216.0);
  const unsigned __int128 prod = (unsigned __int128)tq * tot;
  const unsigned long long target = (unsigned long long)((prod + 16777215u) >> 24);
  if (tid == 0) {
    int kk = 0;
    if (tq > 0 && tot > 0) {
      unsigned long long run = 0;
      while (kk < nJ) {
        run += key[kk] >> 10;
        ++kk;
        if (run >= target) break;
      }
    }
    s_k = kk;
  }
  __syncthreads();
  const int kk = s_k;
  for (int e = tid; e < kk; e += 256) {
    const int J = kXaMaxBlocks - 1 - (int)(key[e] & (kXaMaxBlocks - 1));
    atomicOr(&row_bits[J >> 5], 1u << (J & 31));
  }
  __syncthreads();
  uint32_t* dst = p.bmask + ((size_t)bh * p.nI + I) * p.words;
  for (int w = tid; w < p.words; w += 256) dst[w] = row_bits[w];
  if (p.counts && tid == 0) p.counts[(size_t)bh * p.nI + I] = kk;
}

hipError_t launch_xattn(const XaParams& p, int d, hipStream_t st) {
  const int n_rt = (p.nC + kXaTile - 1) / kXaTile;
  const dim3 g1((unsigned)(p.batch * p.h_q * n_rt));
  const dim3 g2((unsigned)(p.batch * p.h_q * p.nI));
  if (g1.x == 0) return hipSuccess;
  if (d == 128) VS_TRACED(st, "vs_xa_cells", hipLaunchKernelGGL((vs_xa_cells_kernel<128>), g1, dim3(256), 0, st, p));
  else VS_TRACED(st, "vs_xa_cells", hipLaunchKernelGGL((vs_xa_cells_kernel<64>), g1, dim3(256), 0, st, p));
  VS_TRACED(st, "vs_xa_select", hipLaunchKernelGGL(vs_xa_select_kernel, g2, dim3(256), 0, st, p));
  return hipGetLastError();
}

}  // namespace vs
