// vs_fwd.hip — sparse attention forward over the Vertical-Slash support.
//
// MTraining paper note, Algorithm 1 (last step) and Algorithm 2
// (block_bar_sparse_attention_forward): O = softmax(S) V and LSE over the
// support only; online softmax with a running max, a correction factor and
// a running sum ("Ring Attention Paper Analysis", "The Blockwise
// Partitioning Strategy").
//
// gfx950 design.  bf16 inputs: the row-split kernel below (K and V tiles
// staged in LDS by direct loads, shared by the two waves that own a query
// block's 64 rows).  fp32 inputs (vs_fwd_f32_kernel): one workgroup (4 waves)
// per (batch, Q head, 64-row query block); every wave holds Q^T for all 64
// rows in registers and consumes whole 64-key tiles on its own (split over
// keys, not rows), so a K or V row is read by exactly one wave: K goes
// straight from global memory into the A operand of S^T = K Q^T, V is
// transposed through the wave's own LDS region for the A operand of
// O^T += V^T P^T, and P^T feeds the second product from registers
// (slot_perm).  Softmax state is fp32.  The four waves' (max, sum, O) merge
// through LDS at the end.
#include "vs_rows.h"
#include "vs_trace.h"

namespace vs {

// merge_out_and_lse (MTraining paper note, Algorithm 2) of one row's result
// of this call (LSE lc, output O / lg) into a running fp32 result (LSE la,
// output O_acc), as lse_merge does: with mx = max(la, lc), w1 = e^(la - mx),
// w2 = e^(lc - mx), the merged output is (w1 O_acc + w2 O / lg) / (w1 + w2)
// and the merged LSE mx + ln(w1 + w2); two empty results give O = 0 and
// LSE = -inf.  Returns the merged LSE, the weight *a of O_acc and the weight
// *bo of the unnormalised O.
__device__ __forceinline__ float merge_row(float la, float lc, float inv_lg, float* a, float* bo) {
  const float mx = fmaxf(la, lc);
  if (mx == -INFINITY) {
    *a = 0.f;
    *bo = 0.f;
    return -INFINITY;
  }
  const float w1 = expf(la - mx);
  const float w2 = expf(lc - mx);
  const float tot = w1 + w2;
  *a = w1 / tot;
  *bo = w2 / tot * inv_lg;
  return mx + logf(tot);
}

template <int D>
struct FwdWorkerF32 {
  typedef Mfma<float> MF;
  typedef typename MF::frag frag;
  static constexpr int KPL = MF::KPL;
  static constexpr int KC = 2 * KPL;
  static constexpr int NCD = D / KC;   // k chunks over head_dim
  static constexpr int NCT = D / 32;   // 32-channel output tiles
  static constexpr int NCK = 32 / KC;  // k chunks over 32 keys
  // V transposed through registers into [channel][key] (pitch VTP).
  static constexpr int VTP = 32 + 4;
  static constexpr int CG = 4;         // channels per 16-byte load
  static constexpr int KG = 2;         // keys per 8-byte store
  static constexpr int NKG = 32 / KG;
  static constexpr int NVG = NKG * (D / CG) / 64;
  static constexpr int VBUF = D * VTP * 4;  // bytes per staging buffer
  // Rescale the output only when a row max grows by more than 2^8 (in the
  // exp2 domain): exp2(t - m) then stays below 256.
  static constexpr float kRescale = 8.f;

  // The half-tile in flight: K operand and S^T.
  struct Buf {
    frag k[NCD];
    f32x16 s[2];
  };

  frag qf[2][NCD];
  f32x16 o[2][NCT];
  f32x4 vr[NVG * KG];   // raw V rows of the next half-tile
  float m[2], l[2];
  const float* kb;      // K of (batch, kv head): row pos at kb + pos * kvs
  const float* vb;      // V of (batch, kv head): row pos at vb + pos * vvs
  int kvs, vvs;
  char* vt;             // this wave's two staging buffers [2][VBUF]
  float sl2;

  template <class Set>
  __device__ __forceinline__ void load_k(const Set& S, int n, frag (&k)[NCD]) const {
    const int lane = threadIdx.x & 63;
    const int hl = lane >> 5;
    const int l32 = lane & 31;
    // A operand of S^T = K Q^T: slot l32 loads key slot_perm(l32) of the half.
    const unsigned key = S.key_pos(n, slot_perm<KPL>(l32));
    const float* krow = kb + (size_t)key * (size_t)kvs + hl * KPL;
#pragma unroll
    for (int c = 0; c < NCD; ++c) k[c] = load_frag<float>(krow + c * KC);
  }

  // V rows of half n into registers.
  template <class Set>
  __device__ __forceinline__ void load_v(const Set& S, int n) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int g = 0; g < NVG; ++g) {
      const int gi = g * 64 + lane;
      const int kg = gi % NKG;
      const int cg = gi / NKG;
#pragma unroll
      for (int u = 0; u < KG; ++u)
        vr[g * KG + u] = *reinterpret_cast<const f32x4*>(vb + (size_t)S.key_pos(n, kg * KG + u) * (size_t)vvs + cg * CG);
    }
  }

  // Raw V rows transposed into dst[channel][key].
  __device__ __forceinline__ void stage(char* dst) const {
    const int lane = threadIdx.x & 63;
    float* df = reinterpret_cast<float*>(dst);
#pragma unroll
    for (int g = 0; g < NVG; ++g) {
      const int gi = g * 64 + lane;
      const int kg = gi % NKG;
      const int cg = gi / NKG;
#pragma unroll
      for (int c = 0; c < CG; ++c) {
        f32x2 pk;
        pk[0] = vr[g * KG][c];
        pk[1] = vr[g * KG + 1][c];
        *reinterpret_cast<f32x2*>(df + (cg * CG + c) * VTP + kg * KG) = pk;
      }
    }
  }

  // A operand of O^T += V^T P^T: channels 32ct + L%32, keys of k chunk c.
  __device__ __forceinline__ frag vt_frag(const char* src, int ct, int c) const {
    const int lane = threadIdx.x & 63;
    const int hl = lane >> 5;
    const int l32 = lane & 31;
    return reinterpret_cast<const float*>(src)[(32 * ct + l32) * VTP + c * KC + hl * KPL];
  }

  __device__ __forceinline__ void scores(const frag (&k)[NCD], f32x16 (&s)[2]) const {
#pragma unroll
    for (int rg = 0; rg < 2; ++rg) {
      s[rg] = f32x16{0};
#pragma unroll
      for (int c = 0; c < NCD; ++c) s[rg] = MF::mma(k[c], qf[rg][c], s[rg]);
    }
  }

  // Online softmax, first part: masked row maxima of half-tile n and the
  // (rare) rescale of the running state.  Masks the scores in place.
  template <class Set>
  __device__ __forceinline__ void softmax_max(const Set& S, int n, f32x16 (&s)[2]) {
    const int lane = threadIdx.x & 63;
    const int hl = lane >> 5;
    const int l32 = lane & 31;
    if (!S.full(n)) {
#pragma unroll
      for (int rg = 0; rg < 2; ++rg) {
        const int r = 32 * rg + l32;
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (!S.valid(n, reg_row<KPL>(i, hl), r)) s[rg][i] = -INFINITY;
      }
    }
    float tm[2];
#pragma unroll
    for (int rg = 0; rg < 2; ++rg) {
      float mx = s[rg][0];
#pragma unroll
      for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[rg][i]);
      mx = half_max(mx);
      tm[rg] = mx * sl2;
    }
    const bool grow = tm[0] > m[0] + kRescale || tm[1] > m[1] + kRescale;
    if (__any(grow)) {
#pragma unroll
      for (int rg = 0; rg < 2; ++rg) {
        const float mn = fmaxf(m[rg], tm[rg]);
        const float alpha = (m[rg] == -INFINITY) ? 0.f : fast_exp2(m[rg] - mn);
        l[rg] *= alpha;
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) o[rg][ct] *= alpha;
        m[rg] = mn;
      }
    }
  }

  // Online softmax, second part: P = exp2(s*scale*log2e - m), row sums, and
  // P^T of both row groups as B operands.
  __device__ __forceinline__ void softmax_exp(const f32x16 (&s)[2], frag (&pf)[2][NCK]) {
#pragma unroll
    for (int rg = 0; rg < 2; ++rg) {
      const float mu = (m[rg] == -INFINITY) ? 0.f : m[rg];
      float p[16];
      float rs = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        p[i] = fast_exp2(__builtin_fmaf(s[rg][i], sl2, -mu));
        rs += p[i];
      }
      rs = half_sum(rs);
      l[rg] += rs;
#pragma unroll
      for (int c = 0; c < NCK; ++c) pf[rg][c] = MF::pack(&p[c * KPL]);
    }
  }

  __device__ __forceinline__ void pv(const char* src, const frag (&pf)[2][NCK]) {
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
#pragma unroll
      for (int c = 0; c < NCK; ++c) {
        const frag vf = vt_frag(src, ct, c);
#pragma unroll
        for (int rg = 0; rg < 2; ++rg) o[rg][ct] = MF::mma(vf, pf[rg][c], o[rg][ct]);
      }
    }
  }

  // Half-tile n with S^T(n) in b.s and V(n) staged in buffer n & 1.
  // K(n+1) is requested first so that its latency hides behind the softmax
  // of n; V(n+2) is read into registers while S^T(n+1) runs.  Past the end
  // the last half is reloaded and recomputed instead of branching (results
  // unused).
  template <class Set>
  __device__ __forceinline__ void step(const Set& S, int n, int N, Buf& b) {
    frag pf[2][NCK];
    const int n1 = n + 1 < N ? n + 1 : N - 1;
    load_k(S, n1, b.k);
    softmax_max(S, n, b.s);
    softmax_exp(b.s, pf);
    char* cur = vt + (n & 1) * VBUF;
    char* nxt = vt + ((n + 1) & 1) * VBUF;
    stage(nxt);
    load_v(S, n + 2 < N ? n + 2 : N - 1);
    scores(b.k, b.s);
    wave_sync();
    pv(cur, pf);
  }

  template <class Set>
  __device__ __forceinline__ void run(const Set& S) {
    const int N = S.n_halves();
    if (N == 0) return;
    Buf b;
    load_v(S, 0);
    stage(vt);
    load_v(S, N > 1 ? 1 : 0);
    load_k(S, 0, b.k);
    scores(b.k, b.s);
    for (int n = 0; n < N; ++n) step(S, n, N, b);
    __builtin_amdgcn_s_waitcnt(vmcnt_wait(0));
    wave_sync();
  }
};

template <int D>
__global__ __launch_bounds__(kQThreads) void vs_fwd_f32_kernel(AttnParams p) {
  typedef FwdWorkerF32<D> W;
  constexpr int OB_PITCH = D + 4;
  constexpr int OB_BYTES = 64 * OB_PITCH * 4;
  // both V staging buffers of every wave; the output merge afterwards
  constexpr int VT_BYTES = 4 * 2 * W::VBUF;
  constexpr int BUF0 = VT_BYTES > OB_BYTES ? VT_BYTES : OB_BYTES;
  // most of the LDS holds the staging buffers: smaller column batches
  __shared__ QMajorLds<kQThreads, 2 * kQThreads> L;
  __shared__ __attribute__((aligned(16))) char buf[BUF0];
  __shared__ float s_m[4][64];
  __shared__ float s_l[4][64];

  int hb, i_local;
  qmajor_item(p, blockIdx.x, p.nqb, &hb, &i_local);
  const int b = hb / p.h_q;
  const int h = hb % p.h_q;
  const int kvh = h * p.h_kv / p.h_q;
  const RowBlock rb = row_block(p, i_local);
  const int list = (b * p.h_q + h) * p.seg.n_seg + rb.seg;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int hl = lane >> 5;
  const int l32 = lane & 31;

  W wk;
  const float* q = reinterpret_cast<const float*>(p.q);
  const int row0 = i_local * kBlock;  // first row of the block in this batch row
#pragma unroll
  for (int rg = 0; rg < 2; ++rg) {
    const float* qr = q + p.sq.at(b, row0 + 32 * rg + l32, h);
#pragma unroll
    for (int c = 0; c < W::NCD; ++c) wk.qf[rg][c] = load_frag<float>(qr + c * W::KC + hl * W::KPL);
#pragma unroll
    for (int ct = 0; ct < W::NCT; ++ct) wk.o[rg][ct] = f32x16{0};
    wk.m[rg] = -INFINITY;
    wk.l[rg] = 0.f;
  }
  wk.kvs = (int)p.sk.t;
  wk.vvs = (int)p.sv.t;
  wk.kb = reinterpret_cast<const float*>(p.k) + p.sk.at(b, 0, kvh);
  wk.vb = reinterpret_cast<const float*>(p.v) + p.sv.at(b, 0, kvh);
  wk.vt = buf + wave * 2 * W::VBUF;
  wk.sl2 = p.sl2;

  qmajor_drive(p, rb, list, L, qm_bits, wk);

  // Combine the four waves' states: global max, rescaled sums and outputs.
  if (hl == 0) {
    s_m[wave][l32] = wk.m[0];
    s_m[wave][32 + l32] = wk.m[1];
    s_l[wave][l32] = wk.l[0];
    s_l[wave][32 + l32] = wk.l[1];
  }
  __syncthreads();
  float f[2];
#pragma unroll
  for (int rg = 0; rg < 2; ++rg) {
    const int r = 32 * rg + l32;
    float mg = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) mg = fmaxf(mg, s_m[w][r]);
    const float mu = (mg == -INFINITY) ? 0.f : mg;
    f[rg] = fast_exp2(wk.m[rg] - mu);
  }
  float* ob = reinterpret_cast<float*>(buf);
  for (int w = 0; w < 4; ++w) {
    if (wave == w) {
#pragma unroll
      for (int rg = 0; rg < 2; ++rg) {
#pragma unroll
        for (int ct = 0; ct < W::NCT; ++ct) {
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4) {
            const int ch = 32 * ct + 8 * i4 + 4 * hl;
            float* dst = ob + (32 * rg + l32) * OB_PITCH + ch;
            f32x4 v;
#pragma unroll
            for (int u = 0; u < 4; ++u) v[u] = wk.o[rg][ct][4 * i4 + u] * f[rg];
            if (w == 0) {
              *reinterpret_cast<f32x4*>(dst) = v;
            } else {
              f32x4 a = *reinterpret_cast<f32x4*>(dst);
              *reinterpret_cast<f32x4*>(dst) = a + v;
            }
          }
        }
      }
    }
    __syncthreads();
  }
  // Normalise and write O (row-major, coalesced) and LSE, or merge them
  // into the running result.
  __shared__ float s_inv[64];
  __shared__ float s_acc[64];
  if (tid < 64) {
    float mg = -INFINITY;
    for (int w = 0; w < 4; ++w) mg = fmaxf(mg, s_m[w][tid]);
    const float mu = (mg == -INFINITY) ? 0.f : mg;
    float lg = 0.f;
    for (int w = 0; w < 4; ++w) lg += s_l[w][tid] * fast_exp2(s_m[w][tid] - mu);
    const float inv = lg > 0.f ? 1.f / lg : 0.f;
    const float lse = lg > 0.f ? (mg + __log2f(lg)) * kLn2 : -INFINITY;
    float* lp = p.lse + ((size_t)b * p.h_q + h) * p.n_q + (size_t)i_local * kBlock + tid;
    if (p.o_merge) {
      float a, bo;
      *lp = merge_row(*lp, lse, inv, &a, &bo);
      s_acc[tid] = a;
      s_inv[tid] = bo;
    } else {
      *lp = lse;
      s_inv[tid] = inv;
    }
  }
  __syncthreads();
  for (int x = tid; x < 64 * D / 4; x += kQThreads) {
    const int r = x / (D / 4);
    const int c4 = (x % (D / 4)) * 4;
    f32x4 v = *reinterpret_cast<const f32x4*>(ob + r * OB_PITCH + c4) * s_inv[r];
    const size_t off = p.so.at(b, row0 + r, h) + c4;
    float* dst = reinterpret_cast<float*>(p.o_out) + off;
    if (p.o_merge) v += *reinterpret_cast<const f32x4*>(dst) * s_acc[r];
    *reinterpret_cast<f32x4*>(dst) = v;
  }
}

// bf16 forward with the rows split over waves: a workgroup of 2*NS waves
// serves NS key streams; waves w and w + NS take stream w % NS for query
// rows 32 (w / NS) .. +31, so the two waves of a stream share every K and V
// tile and each issues half of its direct loads.  One workgroup barrier per
// half-tile publishes both halves of the loads and frees the other buffer of
// the ring of two.  Each wave keeps Q^T of its 32 rows in registers (about
// 250 registers in all, so two waves fit on a SIMD); per half-tile
// S^T = K Q^T reads K row-wise from LDS, the online softmax runs on the 16
// scores per lane, and O^T += V^T P^T reads V transposed (ds_read_b64_tr_b16)
// with P^T taken from registers (slot_perm).  With NS = 1 (the launched
// form) a workgroup is two waves and needs under 40 KB of LDS, so four
// independent workgroups share a CU: one's index expansion, waits and output
// merge overlap the others' products.

template <int D, int NP = 2>
struct FwdRowsWorker : RowsTiles<D> {
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
  static constexpr int NVW = T::NVL / NP;  // direct loads per half-tile issued by each wave
  static constexpr float kRescale = 8.f;

  frag qf[NCD];   // Q^T of this wave's 32 rows
  f32x16 o[NCT];  // O^T [channel][row]
  float m, l;     // this lane's row: running max (exp2 domain) and sum
  const char* kt[2];      // this stream's K tiles (ring of two)
  const char* vt[2];
  uint32_t kta[2], vta[2];
  float sl2;

  __device__ __forceinline__ frag vt_frag(const char* src, int ct, int c) const { return this->t_frag(src, ct, c); }

  __device__ __forceinline__ void scores(const char* ksrc, f32x16& s) const {
    s = f32x16{0};
#pragma unroll
    for (int c = 0; c < NCD; ++c) s = MF::mma(k_frag(ksrc, c), qf[c], s);
  }

  // Half n of this stream, with S^T(n) in s: masks, online softmax and P V
  // from V tile vc; S^T(n+1) goes into sn from K tile kn meanwhile (the
  // exponentials and these products are independent, so the matrix cores run
  // while the softmax does).
  template <class Set>
  __device__ __forceinline__ void compute(const Set& S, int n, f32x16& s, f32x16& sn, const char* kn,
                                          const char* vc) {
    const int lane = threadIdx.x & 63;
    const int hl = lane >> 5;
    const int r = 32 * rh + (lane & 31);
    if (!S.full(n)) S.template mask<KPL>(n, hl, r, s);
    float mx = s[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[i]);
    const float tm = half_max(mx) * sl2;
    if (__any(tm > m + kRescale)) {
      const float mn = fmaxf(m, tm);
      const float alpha = (m == -INFINITY) ? 0.f : fast_exp2(m - mn);
      l *= alpha;
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) o[ct] *= alpha;
      m = mn;
    }
    const float mu = (m == -INFINITY) ? 0.f : m;
    // Written in issue order, fenced against reordering: each product of
    // S^T(n+1) is followed by a share of the exponentials of half n and one
    // LDS read four products ahead (K rows, then V for the P V products).
    constexpr int NVF = NCT * NCK;
    constexpr int NRD = NCD + NVF;
    constexpr int AHEAD = 4;
    constexpr int EPM = 16 / NCD;
    frag kf[NCD];
    frag vf[NVF];
    auto issue = [&](int i) {
      if (i < NCD) kf[i] = k_frag(kn, i);
      else if (i < NRD) vf[i - NCD] = vt_frag(vc, (i - NCD) % NCT, (i - NCD) / NCT);
    };
#pragma unroll
    for (int i = 0; i < AHEAD; ++i) issue(i);
    float pr[16];
    float rs = 0.f;
    sn = f32x16{0};
    // Wave priorities: the products of S^T(n+1) with the exponentials at 1,
    // the P V products at 2, the barrier and the next tile's loads at 0, so
    // that of the waves of a SIMD the one with matrix-core work issues first
    // and the one closest to finishing its half goes ahead (6.50 -> 6.26 ms
    // with 1 / 1 / 0 at N = 131072, 6.14 -> 5.99 ms with 1 / 2 / 0).
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int c = 0; c < NCD; ++c) {
      sn = MF::mma(kf[c], qf[c], sn);
#pragma unroll
      for (int e = 0; e < EPM; ++e) {
        const int i = c * EPM + e;
        pr[i] = fast_exp2(__builtin_fmaf(s[i], sl2, -mu));
        rs += pr[i];
      }
      issue(c + AHEAD);
      __builtin_amdgcn_sched_barrier(0);
    }
    l += half_sum(rs);
    frag pf[NCK];
#pragma unroll
    for (int c = 0; c < NCK; ++c) pf[c] = MF::pack(&pr[c * KPL]);
    __builtin_amdgcn_s_setprio(2);
#pragma unroll
    for (int j = 0; j < NVF; ++j) {
      o[j % NCT] = MF::mma(vf[j], pf[j / NCT], o[j % NCT]);
      issue(NCD + j + AHEAD);
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
  }

  // Step n (P = n % 2).  K(m) and V(m) live in ring slot m % 2.  Entering,
  // S^T(n) is in s and this wave's loads of K(n+1) and V(n) are in flight;
  // once they have landed the barrier publishes the partner's halves too and
  // tells that every wave is done with K(n) and V(n-1), whose slots take
  // K(n+2) and V(n+1).  Past the end of the stream S^T of the last slot is
  // recomputed instead of branching (results unused).
  template <int P, class Set>
  __device__ __forceinline__ void step(const Set& S, int n, int N, f32x16 (&s)[2]) {
    // this wave's loads have landed and its LDS reads of the previous step
    // have returned before the other waves may overwrite those tiles
    __builtin_amdgcn_s_waitcnt(vmcnt_wait(0) & lgkmcnt_wait0());
    __syncthreads();
    if (n + 2 < N) this->template dma_share<NP>(S, n + 2, kb, this->krb, kta[P]);
    if (n + 1 < N) this->template dma_share<NP>(S, n + 1, vb, this->vrb, vta[P ^ 1]);
    if (n < N) compute(S, n, s[P], s[P ^ 1], kt[P ^ 1], vt[P]);
  }

  // All waves take the same number of steps (the longest stream's), so that
  // every barrier is reached by everyone; a stream with fewer halves idles
  // through its last steps.
  template <class Set>
  __device__ __forceinline__ void run(const Set& S) {
    const int NA = S.n_halves_max();
    if (NA == 0) return;
    const int N = S.n_halves();
    f32x16 s[2];
    if (N > 0) {
      this->template dma_share<NP>(S, 0, kb, this->krb, kta[0]);
      this->template dma_share<NP>(S, 0, vb, this->vrb, vta[0]);
      this->template dma_share<NP>(S, 1, kb, this->krb, kta[1]);
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_wait(NVW));
    __syncthreads();
    if (N > 0) scores(kt[0], s[0]);
    // sets have an even number of halves (two per 64-key tile)
    for (int n = 0; n < NA; n += 2) {
      step<0>(S, n, N, s);
      step<1>(S, n + 1, N, s);
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_wait(0));
  }
};

// PM = kPairBlocks (block selections): the workgroup owns the two query
// blocks of a 128-row block, its four waves rows 0-31 .. 96-127 of the pair
// on one stream, so every K / V tile serves 128 rows (half the loads); past
// an odd block count the second block is absent (its waves compute on the
// first block's rows and store nothing).
template <int D, int NS, int PM = 0>
__global__ __launch_bounds__(128 * NS * (PM ? 2 : 1)) __attribute__((amdgpu_waves_per_eu(2))) void vs_fwd_rows_kernel(AttnParams p) {
  constexpr int QB = PM ? 2 : 1;  // query blocks per workgroup
  static_assert(QB == 1 || NS == 1, "pairs of query blocks run one stream");
  typedef FwdRowsWorker<D, 2 * QB> W;
  constexpr int NT = 128 * NS * QB;
  constexpr int OB_PITCH = D + 4;
  constexpr int OB_BYTES = 64 * OB_PITCH * 4;
  // [ring slot][K, V][stream] tiles
  constexpr int TILES = 2 * 2 * NS * W::TB;
  __shared__ QMajorLds<NT, RowsLdsCfg<NS>::kCols> L;
  __shared__ __attribute__((aligned(16))) char tiles[TILES > OB_BYTES ? TILES : OB_BYTES];
  __shared__ float s_m[NS][64];
  __shared__ float s_l[NS][64];
  __shared__ float s_inv[64];
  __shared__ float s_acc[64];

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
  const __bf16* q = reinterpret_cast<const __bf16*>(p.q);
  const int row0 = i_local * kBlock;  // first row of the block (pair) in this batch row
  const int r = 32 * wk.rh + l32;     // this lane's row of the block (pair)
  // the query block of this wave's rows, and whether it exists
  const int qh = wk.rh >> 1;
  const bool live = QB == 1 || i_local + qh < p.nqb;
  {
    const __bf16* qr = q + p.sq.at(b, row0 + (live ? r : r - kBlock), h);
#pragma unroll
    for (int c = 0; c < W::NCD; ++c) wk.qf[c] = load_frag<__bf16>(qr + c * W::KC + hl * W::KPL);
  }
#pragma unroll
  for (int ct = 0; ct < W::NCT; ++ct) wk.o[ct] = f32x16{0};
  wk.m = -INFINITY;
  wk.l = 0.f;
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

  // One round per query block of the workgroup: combine the streams' states
  // of every row, normalise, write O and LSE (or merge them into the running
  // result).
  for (int u = 0; u < QB; ++u) {
    if (i_local + u >= p.nqb) break;  // uniform: an absent second block
    const bool mine = QB == 1 || qh == u;
    const int rr = r - kBlock * u;    // this lane's row in the round, when mine
    if (mine && hl == 0) {
      s_m[ks][rr] = wk.m;
      s_l[ks][rr] = wk.l;
    }
    __syncthreads();
    float f = 0.f;
    if (mine) {
      float mg = -INFINITY;
#pragma unroll
      for (int w = 0; w < NS; ++w) mg = fmaxf(mg, s_m[w][rr]);
      f = fast_exp2(wk.m - ((mg == -INFINITY) ? 0.f : mg));
    }
    float* ob = reinterpret_cast<float*>(tiles);
    for (int w = 0; w < NS; ++w) {
      if (mine && ks == w) {
#pragma unroll
        for (int ct = 0; ct < W::NCT; ++ct)
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4) {
            float* dst = ob + rr * OB_PITCH + 32 * ct + 8 * i4 + 4 * hl;
            f32x4 v;
#pragma unroll
            for (int x = 0; x < 4; ++x) v[x] = wk.o[ct][4 * i4 + x] * f;
            if (w == 0) *reinterpret_cast<f32x4*>(dst) = v;
            else *reinterpret_cast<f32x4*>(dst) = *reinterpret_cast<f32x4*>(dst) + v;
          }
      }
      __syncthreads();
    }
    const int qrow0 = row0 + kBlock * u;  // first row of the round's query block
    if (tid < 64) {
      float mt = -INFINITY;
      for (int w = 0; w < NS; ++w) mt = fmaxf(mt, s_m[w][tid]);
      const float mu = (mt == -INFINITY) ? 0.f : mt;
      float lg = 0.f;
      for (int w = 0; w < NS; ++w) lg += s_l[w][tid] * fast_exp2(s_m[w][tid] - mu);
      const float inv = lg > 0.f ? 1.f / lg : 0.f;
      const float lse = lg > 0.f ? (mt + __log2f(lg)) * kLn2 : -INFINITY;
      float* lp = p.lse + ((size_t)b * p.h_q + h) * p.n_q + (size_t)qrow0 + tid;
      if (p.o_merge) {
        float a, bo;
        *lp = merge_row(*lp, lse, inv, &a, &bo);
        s_acc[tid] = a;
        s_inv[tid] = bo;
      } else {
        *lp = lse;
        s_inv[tid] = inv;
      }
    }
    __syncthreads();
    for (int x = tid; x < 64 * D / 4; x += NT) {
      const int orow = x / (D / 4);
      const int c4 = (x % (D / 4)) * 4;
      f32x4 v = *reinterpret_cast<const f32x4*>(ob + orow * OB_PITCH + c4) * s_inv[orow];
      const size_t off = p.so.at(b, qrow0 + orow, h) + c4;
      if (p.o_f32) {
        float* dst = reinterpret_cast<float*>(p.o_out) + off;
        if (p.o_merge) v += *reinterpret_cast<const f32x4*>(dst) * s_acc[orow];
        *reinterpret_cast<f32x4*>(dst) = v;
      } else {
        bf16x4 w4;
#pragma unroll
        for (int x4 = 0; x4 < 4; ++x4) w4[x4] = (__bf16)v[x4];
        *reinterpret_cast<bf16x4*>(reinterpret_cast<__bf16*>(p.o_out) + off) = w4;
      }
    }
    if (QB > 1) __syncthreads();  // the next round reuses the staging buffers
  }
}


hipError_t launch_fwd(const AttnParams& p, int dtype_bf16, int d, hipStream_t st) {
  const dim3 grid((unsigned)(p.batch * p.h_q * p.nqb));
  if (grid.x == 0) return hipSuccess;
  const size_t dyn = qmajor_bits_bytes(p);
  if (dtype_bf16 && p.bmask) {
    // block selections: pairs of query blocks
    const dim3 gp((unsigned)(p.batch * p.h_q * ((p.nqb + 1) / 2)));
    if (d == 128) VS_TRACED(st, "vs_fwd", hipLaunchKernelGGL((vs_fwd_rows_kernel<128, 1, kPairBlocks>), gp, dim3(256), dyn, st, p));
    else VS_TRACED(st, "vs_fwd", hipLaunchKernelGGL((vs_fwd_rows_kernel<64, 1, kPairBlocks>), gp, dim3(256), dyn, st, p));
  } else if (dtype_bf16 && d == 128) VS_TRACED(st, "vs_fwd", hipLaunchKernelGGL((vs_fwd_rows_kernel<128, 1>), grid, dim3(128), dyn, st, p));
  else if (dtype_bf16) VS_TRACED(st, "vs_fwd", hipLaunchKernelGGL((vs_fwd_rows_kernel<64, 1>), grid, dim3(128), dyn, st, p));
  else if (d == 128) VS_TRACED(st, "vs_fwd", hipLaunchKernelGGL((vs_fwd_f32_kernel<128>), grid, dim3(kQThreads), dyn, st, p));
  else VS_TRACED(st, "vs_fwd", hipLaunchKernelGGL((vs_fwd_f32_kernel<64>), grid, dim3(kQThreads), dyn, st, p));
  return hipGetLastError();
}

}  // namespace vs
