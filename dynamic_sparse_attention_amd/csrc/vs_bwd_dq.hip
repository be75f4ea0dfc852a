// vs_bwd_dq.hip — dQ of the sparse backward, query-major, bf16 inputs.
//
// MTraining §3.2 Eq. 1-2 and the paper note's Appendix B.1:
// dQ = scale * dS K with dS = P * (dP - delta), P = exp(S - LSE) recomputed
// from the final LSE and dP = dO V^T, over the forward's support.
//
// Query-major, with the walk of the forward: a workgroup owns a query block
// (its two waves rows 0-31 and 32-63) and walks the block's slash tiles and
// its uncovered vertical columns, K and V staged in LDS by direct loads and
// shared by the two waves.
#include "vs_rows.h"
#include "vs_trace.h"

namespace vs {

// Row-split dQ: a workgroup of 2*NS waves serves NS key streams, the two
// waves of a stream own rows 0-31 and 32-63 and share its K and V tiles in
// LDS (both read row-wise for S^T = K Q^T and dP^T = V dO^T, K also
// transposed for dQ^T += K^T dS^T).  Each wave holds Q^T, dO^T and dQ^T of
// its 32 rows (about 235 registers), so with NS = 1 (the launched form: two
// waves, under 40 KB of LDS) four independent workgroups share a CU.
template <int D, int NP = 2>
struct DqRowsWorker : RowsTiles<D> {
  typedef RowsTiles<D> T;
  typedef typename T::MF MF;
  typedef typename T::frag frag;
  using T::KPL;
  using T::NCD;
  using T::NCT;
  using T::NCK;
  using T::kb;
  using T::vb;
  using T::rh;
  using T::k_frag;
  using T::t_frag;
  static constexpr int NVW = T::NVL / NP;  // direct loads per half-tile issued by each wave

  frag qf[NCD];     // Q^T of this wave's 32 rows
  frag dof[NCD];    // dO^T
  f32x16 dq[NCT];   // dQ^T [channel][row]
  f32x16 s, dp;     // S^T, dP^T of the current half
  float lse2;       // this lane's row: LSE * log2(e), +inf for an empty row
  float dl;         // delta
  const char* kt[2];  // this stream's tiles (rings of two)
  const char* vt[2];
  uint32_t kta[2], vta[2];
  float sl2;

  __device__ __forceinline__ void scores(const char* ksrc, const char* vsrc) {
    s = f32x16{0};
    dp = f32x16{0};
#pragma unroll
    for (int c = 0; c < NCD; ++c) {
      s = MF::mma(k_frag(ksrc, c), qf[c], s);
      dp = MF::mma(k_frag(vsrc, c), dof[c], dp);
    }
  }

  // dS^T of half n as bf16 B operands: P = exp2(S log2(e) scale - LSE log2(e)),
  // dS = P (dP - delta); masked and empty-row entries give P = 0.
  template <class Set>
  __device__ __forceinline__ void dscores(const Set& S, int n, frag (&dsf)[NCK]) {
    const int lane = threadIdx.x & 63;
    const int hl = lane >> 5;
    const int r = 32 * rh + (lane & 31);
    if (!S.full(n)) S.template mask<KPL>(n, hl, r, s);
    float ds[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float pr = fast_exp2(__builtin_fmaf(s[i], sl2, -lse2));
      ds[i] = pr * (dp[i] - dl);
    }
#pragma unroll
    for (int c = 0; c < NCK; ++c) dsf[c] = MF::pack(&ds[c * KPL]);
  }

  // Step n (P = n % 2).  K(m) and V(m) live in ring slot m % 2.  Entering,
  // S^T(n), dP^T(n) are in s, dp and this wave's loads of K(n+1), V(n+1) are
  // in flight.  dS(n) and the dQ products of half n (K(n) transposed) come
  // first; the barrier then publishes K(n+1), V(n+1) and tells that every
  // wave is done with K(n) and V(n), whose slots take K(n+2), V(n+2); S^T and
  // dP^T of n+1 follow.
  template <int P, class Set>
  __device__ __forceinline__ void step(const Set& S, int n, int N) {
    // Wave priorities: dS at 1, its dQ products at 2, the barrier and the
    // loads at 0, the next half's S and dP products at 1 (8.06 -> 7.97 ms
    // at N = 131072).
    if (n < N) {
      frag dsf[NCK];
      __builtin_amdgcn_s_setprio(1);
      dscores(S, n, dsf);
      __builtin_amdgcn_s_setprio(2);
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int c = 0; c < NCK; ++c) dq[ct] = MF::mma(t_frag(kt[P], ct, c), dsf[c], dq[ct]);
      __builtin_amdgcn_s_setprio(0);
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_wait(0) & lgkmcnt_wait0());
    __syncthreads();
    if (n + 2 < N) {
      this->template dma_share<NP>(S, n + 2, kb, this->krb, kta[P]);
      this->template dma_share<NP>(S, n + 2, vb, this->vrb, vta[P]);
    }
    __builtin_amdgcn_s_setprio(1);
    if (n + 1 < N) scores(kt[P ^ 1], vt[P ^ 1]);
    __builtin_amdgcn_s_setprio(0);
  }

  // All waves take the same number of steps (the longest stream's), so that
  // every barrier is reached by everyone.
  template <class Set>
  __device__ __forceinline__ void run(const Set& S) {
    const int NA = S.n_halves_max();
    if (NA == 0) return;
    const int N = S.n_halves();
    if (N > 0) {
      this->template dma_share<NP>(S, 0, kb, this->krb, kta[0]);
      this->template dma_share<NP>(S, 0, vb, this->vrb, vta[0]);
      this->template dma_share<NP>(S, 1, kb, this->krb, kta[1]);
      this->template dma_share<NP>(S, 1, vb, this->vrb, vta[1]);
    }
    // this wave's loads of K(0), V(0) have landed (K(1), V(1) may not have)
    __builtin_amdgcn_s_waitcnt(vmcnt_wait(2 * NVW));
    __syncthreads();
    if (N > 0) scores(kt[0], vt[0]);
    // sets have an even number of halves (two per 64-key tile)
    for (int n = 0; n < NA; n += 2) {
      step<0>(S, n, N);
      step<1>(S, n + 1, N);
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_wait(0));
  }
};

// PM = kPairBlocks (block selections): the two query blocks of a 128-row
// block in one workgroup, four waves on one stream (half the K / V loads);
// an absent second block's waves compute on the first block's rows and
// store nothing.
template <int D, int NS, int PM = 0>
__global__ __launch_bounds__(128 * NS * (PM ? 2 : 1)) __attribute__((amdgpu_waves_per_eu(2))) void vs_bwd_dq_rows_kernel(AttnParams p) {
  constexpr int QB = PM ? 2 : 1;  // query blocks per workgroup
  static_assert(QB == 1 || NS == 1, "pairs of query blocks run one stream");
  typedef DqRowsWorker<D, 2 * QB> W;
  constexpr int NT = 128 * NS * QB;
  constexpr int OB_PITCH = D + 4;
  constexpr int OB_BYTES = 64 * OB_PITCH * 4;
  // [ring slot][K, V][stream] tiles
  constexpr int TILES = 2 * 2 * NS * W::TB;
  __shared__ QMajorLds<NT, RowsLdsCfg<NS>::kCols> L;
  __shared__ __attribute__((aligned(16))) char tiles[TILES > OB_BYTES ? TILES : OB_BYTES];

  int hb, i_local;
  qmajor_item(p, blockIdx.x, (p.nqb + QB - 1) / QB, &hb, &i_local);
  i_local *= QB;
  const int b = hb / p.h_q;
  const int h = hb % p.h_q;
  const int kvh = h * p.h_kv / p.h_q;
  const RowBlock rb = row_block(p, i_local);
  const int list = (b * p.h_q + h) * p.seg.n_seg + rb.seg;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int ks = wave % NS;
  const int lane = tid & 63;
  const int hl = lane >> 5;
  const int l32 = lane & 31;

  W wk;
  wk.rh = __builtin_amdgcn_readfirstlane(wave / NS);
  const int r = 32 * wk.rh + l32;  // this lane's row of the block (pair)
  const int qh = wk.rh >> 1;       // the query block of this wave's rows
  const bool live = QB == 1 || i_local + qh < p.nqb;
  const int rl = live ? r : r - kBlock;  // the row it reads (an absent block's waves read the first block's)
  const __bf16* q = reinterpret_cast<const __bf16*>(p.q);
  const __bf16* dout = reinterpret_cast<const __bf16*>(p.dout);
  const int row0 = i_local * kBlock;  // first row of the block (pair) in this batch row
  {
    const size_t qoff = p.sq.at(b, row0 + rl, h) + hl * W::KPL;
    const size_t doff = p.sdo.at(b, row0 + rl, h) + hl * W::KPL;
    const size_t roff = p.so.at(b, row0 + rl, h) + hl * W::KPL;  // O, for delta
#pragma unroll
    for (int c = 0; c < W::NCD; ++c) {
      wk.qf[c] = load_frag<__bf16>(q + qoff + c * W::KC);
      wk.dof[c] = load_frag<__bf16>(dout + doff + c * W::KC);
    }
    const size_t li = ((size_t)b * p.h_q + h) * p.n_q + (size_t)i_local * kBlock + rl;
    const float lse = p.lse[li];
    wk.lse2 = (lse == -INFINITY) ? INFINITY : lse * kLog2e;
    if (p.delta_out) {
      // delta = rowsum(dO * O) of this lane's row (Eq. 1), from the dO^T
      // fragments already in registers; lanes L and L + 32 hold the two
      // halves of every channel chunk of one row.
      float acc = 0.f;
      if (p.o_f32) {
        const float* o = reinterpret_cast<const float*>(p.o) + roff;
#pragma unroll
        for (int c = 0; c < W::NCD; ++c) {
          const f32x4 a = *reinterpret_cast<const f32x4*>(o + c * W::KC);
          const f32x4 a2 = *reinterpret_cast<const f32x4*>(o + c * W::KC + 4);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            acc = __builtin_fmaf(a[j], (float)wk.dof[c][j], acc);
            acc = __builtin_fmaf(a2[j], (float)wk.dof[c][4 + j], acc);
          }
        }
      } else {
        const __bf16* o = reinterpret_cast<const __bf16*>(p.o) + roff;
#pragma unroll
        for (int c = 0; c < W::NCD; ++c) {
          const bf16x8 a = load_frag<__bf16>(o + c * W::KC);
#pragma unroll
          for (int j = 0; j < 8; ++j) acc = __builtin_fmaf((float)a[j], (float)wk.dof[c][j], acc);
        }
      }
      acc += __shfl_xor(acc, 32, 64);
      wk.dl = acc;
      if (hl == 0 && live) p.delta_out[li] = acc;
    } else {
      wk.dl = p.delta[li];
    }
    if (p.lse2_out && hl == 0 && live) p.lse2_out[li] = wk.lse2;
  }
#pragma unroll
  for (int ct = 0; ct < W::NCT; ++ct) wk.dq[ct] = f32x16{0};
  wk.krb = (uint32_t)(p.sk.t * 2);
  wk.vrb = (uint32_t)(p.sv.t * 2);
  wk.kb = reinterpret_cast<const __bf16*>(p.k) + p.sk.at(b, 0, kvh);
  wk.vb = reinterpret_cast<const __bf16*>(p.v) + p.sv.at(b, 0, kvh);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    wk.kt[i] = tiles + ((i * 2 + 0) * NS + ks) * W::TB;
    wk.vt[i] = tiles + ((i * 2 + 1) * NS + ks) * W::TB;
    wk.kta[i] = lds_addr(wk.kt[i]);
    wk.vta[i] = lds_addr(wk.vt[i]);
  }
  wk.sl2 = p.sl2;
  wk.init_offsets();

  qmajor_drive<NS, PM>(p, rb, list, L, qm_bits, wk);

  // One round per query block of the workgroup: sum the streams' dQ^T of
  // every row, then scale and store (or add).
  float* ob = reinterpret_cast<float*>(tiles);
  for (int u = 0; u < QB; ++u) {
    if (i_local + u >= p.nqb) break;  // uniform: an absent second block
    const bool mine = QB == 1 || qh == u;
    const int rr = r - kBlock * u;
    for (int w = 0; w < NS; ++w) {
      if (mine && ks == w) {
#pragma unroll
        for (int ct = 0; ct < W::NCT; ++ct)
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4) {
            float* dst = ob + rr * OB_PITCH + 32 * ct + 8 * i4 + 4 * hl;
            f32x4 v;
#pragma unroll
            for (int x = 0; x < 4; ++x) v[x] = wk.dq[ct][4 * i4 + x];
            if (w == 0) *reinterpret_cast<f32x4*>(dst) = v;
            else *reinterpret_cast<f32x4*>(dst) = *reinterpret_cast<f32x4*>(dst) + v;
          }
      }
      __syncthreads();
    }
    const int qrow0 = row0 + kBlock * u;
    for (int x = tid; x < 64 * D / 4; x += NT) {
      const int orow = x / (D / 4);
      const int c4 = (x % (D / 4)) * 4;
      const f32x4 v = *reinterpret_cast<const f32x4*>(ob + orow * OB_PITCH + c4) * p.scale;
      float* dst = p.dq + (((size_t)b * p.n_q + qrow0 + orow) * p.h_q + h) * D + c4;
      if (p.dq_accumulate) *reinterpret_cast<f32x4*>(dst) = *reinterpret_cast<f32x4*>(dst) + v;
      else *reinterpret_cast<f32x4*>(dst) = v;
    }
    if (QB > 1) __syncthreads();  // the next round reuses the staging buffer
  }
}

hipError_t launch_bwd_dq_bf16(const AttnParams& p, int d, hipStream_t st) {
  const dim3 gq((unsigned)(p.batch * p.h_q * p.nqb));
  if (gq.x == 0) return hipSuccess;
  const size_t dyn = qmajor_bits_bytes(p);
  if (p.bmask) {
    // block selections: pairs of query blocks
    const dim3 gp((unsigned)(p.batch * p.h_q * ((p.nqb + 1) / 2)));
    if (d == 128) VS_TRACED(st, "vs_bwd_dq", hipLaunchKernelGGL((vs_bwd_dq_rows_kernel<128, 1, kPairBlocks>), gp, dim3(256), dyn, st, p));
    else VS_TRACED(st, "vs_bwd_dq", hipLaunchKernelGGL((vs_bwd_dq_rows_kernel<64, 1, kPairBlocks>), gp, dim3(256), dyn, st, p));
  } else if (d == 128) VS_TRACED(st, "vs_bwd_dq", hipLaunchKernelGGL((vs_bwd_dq_rows_kernel<128, 1>), gq, dim3(128), dyn, st, p));
  else VS_TRACED(st, "vs_bwd_dq", hipLaunchKernelGGL((vs_bwd_dq_rows_kernel<64, 1>), gq, dim3(128), dyn, st, p));
  return hipGetLastError();
}

}  // namespace vs
