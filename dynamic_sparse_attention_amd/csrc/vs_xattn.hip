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
// gfx950 design.  vs_xa_cells_kernel: the cell logits of one (batch, Q
// head) are a contraction over S * d = 16 * 128 (the sample offset u and the
// channel), i.e. a GEMM Z = Qc Kc^T restricted to the causal lower triangle
// of the cell grid.  One workgroup (4 waves, 2 x 2, each 64 x 64 cells) takes
// a tile of 128 cell rows x 128 cell columns at or below the diagonal and
// walks the contraction in stages of one offset u and 64 channels: the 128
// sampled Q rows 16 A + u and the 128 sampled K rows 16 C + 15 - u of the
// stage (16 KB each) arrive in LDS by direct global -> LDS loads, double
// buffered, with each row's 16-byte chunks at chunk ^ ((row / 2) % 8) so that
// every 16-lane pass of an operand read hits 16 different bank groups; the
// matrix cores (v_mfma_f32_32x32x16_bf16, cell columns as the A operand, cell
// rows as B) accumulate in registers.  The epilogue turns each lane's 4 x 4
// column values into log-sum-exps of the 8 cells of a key block (two lanes
// hold the two halves) and stores them column-major in the key block, so 32
// consecutive cell rows store together.  vs_xa_select_kernel: one workgroup
// per (batch, Q head, query block) reads the log-sum-exps of its 8 cell rows
// for every key block J <= I, forms each row's log-sum-exp, the block scores
// s[I, J] = sum over the rows of 2^(lse[A, J] - lse[A]), takes integer masses
// rint(s * 2^50) (exact and the same in every run), sorts the (mass, index)
// keys with a bitonic sort in LDS and keeps the shortest prefix whose mass
// reaches ceil(rint(t * 2^24) * total / 2^24).
#include "vs_attn_common.h"
#include "vs_trace.h"
#include "vs_xattn_params.h"

namespace vs {

constexpr int kXaStride = 16;      // S
constexpr int kXaBlock = 128;      // block side (tokens)
constexpr int kXaCpb = kXaBlock / kXaStride;  // cells per block side: 8
constexpr int kXaTile = 128;       // cell rows / columns per workgroup tile
constexpr int kXaChan = 64;        // channels per stage
constexpr int kXaRowBytes = kXaChan * 2;           // 128: one sampled row of a stage
constexpr int kXaOpBytes = kXaTile * kXaRowBytes;  // 16 KB: one operand of a stage

// byte offset of chunk c (16 bytes) of row r of a stage operand in LDS
__device__ __forceinline__ int xa_off(int r, int c) { return r * kXaRowBytes + 16 * (c ^ ((r >> 1) & 7)); }

struct __attribute__((aligned(16))) XaStage {
  char q[kXaOpBytes];  // sampled Q rows of the tile's cell rows
  char k[kXaOpBytes];  // sampled K rows of the tile's cell columns
};

// Loads of stage st (offset u = st / (D / 64), channels 64 * (st % (D / 64)))
// into B: 32 direct loads of 1 KB (8 rows each), 8 per wave.  Lane L of the
// load for rows 8 t .. 8 t + 7 fills LDS chunk L % 8 of row 8 t + L / 8, so
// it fetches that row's chunk (L % 8) ^ ((row / 2) % 8).
template <int D>
__device__ __forceinline__ void xa_stage_dma(const XaParams& p, XaStage& B, const __bf16* qb, const __bf16* kb,
                                             int A0, int C0, int st) {
  constexpr int SPU = D / kXaChan;  // stages per offset
  const int u = st / SPU;
  const int ch0 = kXaChan * (st % SPU);
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rsub = lane >> 3;
#pragma unroll
  for (int t0 = 0; t0 < 8; ++t0) {
    const int t = w * 8 + t0;          // 0..31: 16 Q loads, then 16 K loads
    const int op = t >> 4;             // 0: Q, 1: K
    const int row = 8 * (t & 15) + rsub;
    const int chunk = (lane & 7) ^ ((row >> 1) & 7);
    const __bf16* src;
    if (op == 0) {
      const int A = min(A0 + row, p.nC - 1);
      src = qb + (size_t)(kXaStride * A + u) * p.sq.t + ch0 + 8 * chunk;
    } else {
      const int C = min(C0 + row, p.nC - 1);
      src = kb + (size_t)(kXaStride * C + kXaStride - 1 - u) * p.sk.t + ch0 + 8 * chunk;
    }
    dma_lds16(src, (op == 0 ? B.q : B.k) + 1024 * (t & 15));
  }
}

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void vs_xa_cells_kernel(XaParams p) {
  typedef Mfma<__bf16> MF;
  typedef MF::frag frag;
  constexpr int NST = kXaStride * D / kXaChan;  // stages
  __shared__ XaStage buf[2];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, hl = lane >> 5, l32 = lane & 31;
  const int wr = wave >> 1, wc = wave & 1;  // this wave's 64 x 64 quarter
  // tile (ta, tc), tc <= ta, of head bh: triangle index t = ta (ta + 1) / 2 + tc
  const int nt = (p.nC + kXaTile - 1) / kXaTile;
  const int per_head = nt * (nt + 1) / 2;
  const int bh = blockIdx.x / per_head;
  const int t = blockIdx.x % per_head;
  int ta = (int)((sqrtf(8.f * (float)t + 1.f) - 1.f) * 0.5f);
  while (ta * (ta + 1) / 2 > t) --ta;
  while ((ta + 1) * (ta + 2) / 2 <= t) ++ta;
  const int tc = t - ta * (ta + 1) / 2;
  const int b = bh / p.h_q, h = bh % p.h_q;
  const int kvh = h * p.h_kv / p.h_q;
  const int A0 = ta * kXaTile, C0 = tc * kXaTile;
  const __bf16* qb = p.q + p.sq.at(b, 0, h);
  const __bf16* kb = p.k + p.sk.at(b, 0, kvh);

  f32x16 acc[2][2];  // [row sub-tile i][column sub-tile j]: C[col][row]
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{0};

  xa_stage_dma<D>(p, buf[0], qb, kb, A0, C0, 0);
  for (int st = 0; st < NST; ++st) {
    // this wave's loads of stage st have landed and its reads of stage st-1
    // have returned; the barrier publishes every wave's loads and frees the
    // other buffer
    __builtin_amdgcn_s_waitcnt(vmcnt_wait(0) & lgkmcnt_wait0());
    __syncthreads();
    if (st + 1 < NST) xa_stage_dma<D>(p, buf[(st + 1) & 1], qb, kb, A0, C0, st + 1);
    const XaStage& B = buf[st & 1];
#pragma unroll
    for (int ks = 0; ks < kXaChan / 16; ++ks) {
      const int c = 2 * ks + hl;
      frag qf[2], kf[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = 64 * wr + 32 * i + l32;
        qf[i] = *reinterpret_cast<const frag*>(B.q + xa_off(r, c));
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int r = 64 * wc + 32 * j + l32;
        kf[j] = *reinterpret_cast<const frag*>(B.k + xa_off(r, c));
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = MF::mma(kf[j], qf[i], acc[i][j]);
    }
  }

  // Epilogue: register e of acc[i][j] holds cell row A0 + 64 wr + 32 i + l32,
  // cell column C0 + 64 wc + 32 j + c_row(e, hl); the 4 registers 4q .. 4q+3
  // are columns 8q + 4hl .. +3, half of key block (C0 + 64 wc + 32 j) / 8 + q,
  // whose other half the lane ^ 32 holds.
  const float zs = p.sl2 / kXaStride;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int A = A0 + 64 * wr + 32 * i + l32;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int Cb = C0 + 64 * wc + 32 * j;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float z[4];
        float mx = -INFINITY;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int C = Cb + 8 * q + 4 * hl + e;
          z[e] = (C <= A && C < p.nC) ? acc[i][j][4 * q + e] * zs : -INFINITY;
          mx = fmaxf(mx, z[e]);
        }
        const float mu = mx == -INFINITY ? 0.f : mx;
        float sm = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) sm += fast_exp2(z[e] - mu);
        // both halves' (max, sum): after the swaps m_lo / s_lo hold the lower
        // half's, m_hi / s_hi the upper half's, in every lane
        float m_lo = mx, m_hi = mx, s_lo = sm, s_hi = sm;
        swap_halves(m_lo, m_hi);
        swap_halves(s_lo, s_hi);
        const float mm = fmaxf(m_lo, m_hi);
        const float mmu = mm == -INFINITY ? 0.f : mm;
        const float tot = (m_lo == -INFINITY ? 0.f : s_lo * fast_exp2(m_lo - mmu)) +
                          (m_hi == -INFINITY ? 0.f : s_hi * fast_exp2(m_hi - mmu));
        const float lse = tot > 0.f ? mmu + __log2f(tot) : -INFINITY;
        const int J = Cb / kXaCpb + q;
        if ((q >> 1) == hl && A < p.nC && J < p.nI)
          p.cell_lse[((size_t)bh * p.nI + J) * p.nC + A] = lse;
      }
    }
  }
}

// Bitonic sort of the first ns (a power of two) 64-bit keys in LDS,
// descending, by 256 threads.
__device__ __forceinline__ void bitonic_desc(unsigned long long* key, int ns) {
  for (int size = 2; size <= ns; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int t = threadIdx.x; t < ns / 2; t += 256) {
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
  constexpr int JPT = kXaMaxBlocks / 256;  // key blocks per thread
  __shared__ unsigned long long key[kXaMaxBlocks];
  __shared__ unsigned long long wsum[4];
  __shared__ float red_m[4][kXaCpb];
  __shared__ float red_s[4][kXaCpb];
  __shared__ uint32_t row_bits[kXaMaxBlocks / 32];
  __shared__ int s_k;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int I = blockIdx.x % p.nI;
  const int bh = blockIdx.x / p.nI;
  const int nJ = I + 1;
  const int a_lo = I * kXaCpb;
  const int na = min(kXaCpb, p.nC - a_lo);  // cell rows of this query block
  // log-sum-exps of the block's cell rows over this thread's key blocks
  // J = tid + 256 jj (all 1024 key slots, -inf past the causal ones)
  float v[JPT][kXaCpb];
#pragma unroll
  for (int jj = 0; jj < JPT; ++jj) {
    const int J = tid + 256 * jj;
    const float* src = p.cell_lse + ((size_t)bh * p.nI + min(J, p.nI - 1)) * p.nC + a_lo;
#pragma unroll
    for (int a = 0; a < kXaCpb; ++a) v[jj][a] = (J < nJ && a < na) ? src[a] : -INFINITY;
  }
  // each cell row's log-sum-exp over its key blocks J <= I (the normaliser of
  // its softmax over the cells C <= A): block-wide maximum, then sum
  float rm[kXaCpb], rl[kXaCpb];
#pragma unroll
  for (int a = 0; a < kXaCpb; ++a) {
    float x = -INFINITY;
#pragma unroll
    for (int jj = 0; jj < JPT; ++jj) x = fmaxf(x, v[jj][a]);
    for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
    rm[a] = x;
  }
  if (lane == 0) {
#pragma unroll
    for (int a = 0; a < kXaCpb; ++a) red_m[wave][a] = rm[a];
  }
  __syncthreads();
#pragma unroll
  for (int a = 0; a < kXaCpb; ++a) {
    rm[a] = fmaxf(fmaxf(red_m[0][a], red_m[1][a]), fmaxf(red_m[2][a], red_m[3][a]));
    const float mu = rm[a] == -INFINITY ? 0.f : rm[a];
    float x = 0.f;
#pragma unroll
    for (int jj = 0; jj < JPT; ++jj) x += v[jj][a] == -INFINITY ? 0.f : fast_exp2(v[jj][a] - mu);
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
    rl[a] = x;
  }
  if (lane == 0) {
#pragma unroll
    for (int a = 0; a < kXaCpb; ++a) red_s[wave][a] = rl[a];
  }
  __syncthreads();
#pragma unroll
  for (int a = 0; a < kXaCpb; ++a) {
    const float sum = red_s[0][a] + red_s[1][a] + red_s[2][a] + red_s[3][a];
    rl[a] = sum > 0.f ? (rm[a] == -INFINITY ? 0.f : rm[a]) + __log2f(sum) : -INFINITY;
  }
  // block scores and their integer masses (exact multiples of 2^-50; s <= 8)
  unsigned long long tot = 0;
#pragma unroll
  for (int jj = 0; jj < JPT; ++jj) {
    const int J = tid + 256 * jj;
    unsigned long long w = 0;
    if (J < nJ) {
      float sc = 0.f;
#pragma unroll
      for (int a = 0; a < kXaCpb; ++a)
        if (v[jj][a] != -INFINITY) sc += fast_exp2(v[jj][a] - rl[a]);
      if (p.scores) p.scores[((size_t)bh * p.nI + I) * p.nI + J] = sc;
      w = (unsigned long long)rint((double)sc * 1125899906842624.0);  // 2^50
    }
    tot += w;
    // (mass, lowest index first): sorted descending by mass, then by 1023 - J
    key[J] = (w << 10) | (unsigned long long)(kXaMaxBlocks - 1 - J);
  }
  for (int o = 32; o > 0; o >>= 1) tot += __shfl_xor(tot, o, 64);
  if (lane == 0) wsum[wave] = tot;
  for (int w = tid; w < kXaMaxBlocks / 32; w += 256) row_bits[w] = 0u;
  if (tid == 0) s_k = nJ;
  __syncthreads();
  tot = wsum[0] + wsum[1] + wsum[2] + wsum[3];
  // the real keys are the first nJ; sort the smallest power of two holding them
  int ns = 2;
  while (ns < nJ) ns <<= 1;
  bitonic_desc(key, ns);
  // target = ceil(rint(t * 2^24) * total / 2^24), t clamped to [0, 1]
  float t = p.threshold;
  t = (t > 0.f) ? fminf(t, 1.f) : 0.f;
  const unsigned long long tq = (unsigned long long)rint((double)t * 16777216.0);
  const unsigned __int128 prod = (unsigned __int128)tq * tot;
  const unsigned long long target = (unsigned long long)((prod + 16777215u) >> 24);
  // the shortest prefix of the sorted masses reaching the target: a
  // block-wide inclusive scan over 4 positions per thread, then the first
  // position whose running mass reaches it
  unsigned long long run4[4], acc = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int pos = 4 * tid + e;
    acc += pos < nJ ? (key[pos] >> 10) : 0ull;
    run4[e] = acc;
  }
  unsigned long long x = acc;
  for (int o = 1; o < 64; o <<= 1) {
    const unsigned long long y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  __syncthreads();  // every wave has read its keys; wsum is free again
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  unsigned long long before = x - acc;
  for (int w = 0; w < wave; ++w) before += wsum[w];
  if (tq > 0 && tot > 0) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int pos = 4 * tid + e;
      if (pos < nJ && before + run4[e] >= target) {
        atomicMin(&s_k, pos + 1);
        break;
      }
    }
  } else if (tid == 0) {
    s_k = 0;
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
  const int nt = (p.nC + kXaTile - 1) / kXaTile;
  const dim3 g1((unsigned)(p.batch * p.h_q * (nt * (nt + 1) / 2)));
  const dim3 g2((unsigned)(p.batch * p.h_q * p.nI));
  if (g1.x == 0) return hipSuccess;
  if (d == 128) VS_TRACED(st, "vs_xa_cells", hipLaunchKernelGGL((vs_xa_cells_kernel<128>), g1, dim3(256), 0, st, p));
  else VS_TRACED(st, "vs_xa_cells", hipLaunchKernelGGL((vs_xa_cells_kernel<64>), g1, dim3(256), 0, st, p));
  VS_TRACED(st, "vs_xa_select", hipLaunchKernelGGL(vs_xa_select_kernel, g2, dim3(256), 0, st, p));
  return hipGetLastError();
}

}  // namespace vs
