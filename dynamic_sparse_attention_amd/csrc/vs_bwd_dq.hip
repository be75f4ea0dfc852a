// vs_bwd_dq.hip — dQ of the sparse backward, query-major, bf16 inputs.
//
// MTraining §3.2 Eq. 1-2 and the paper note's Appendix B.1:
// dQ = scale * dS K with dS = P * (dP - delta), P = exp(S - LSE) recomputed
// from the final LSE and dP = dO V^T, over the forward's support.
//
// Same walk and wave split as the forward (each wave owns all 64 rows and a
// share of the 32-key half-tiles).  Per half-tile the K rows arrive by direct
// global -> LDS loads into a row-major, chunk-swizzled buffer; the A operand
// of S^T = K Q^T is read from it row-wise and the A operand of
// dQ^T += K^T dS^T transposed (ds_read_b64_tr_b16), so K is fetched once.  V
// goes straight to registers as the A operand of dP^T = V dO^T.  The loads
// of half n+1 are issued at the start of step n, and S^T, dP^T of n+1 are
// computed after the dQ products of n.
#include "vs_rows.h"
#include "vs_trace.h"

namespace vs {

template <int D>
struct DqWorkerB {
  typedef Mfma<__bf16> MF;
  typedef MF::frag frag;
  static constexpr int KPL = 8, KC = 16, NCK = 2;
  static constexpr int NCD = D / KC;
  static constexpr int NCT = D / 32;
  static constexpr int CPR = D / 8;           // 16-byte chunks per row
  static constexpr int RPI = 64 / CPR;        // rows per 1 KiB direct-load instruction
  static constexpr int NVL = 32 / RPI;        // direct loads per half-tile
  static constexpr int HBYTES = 32 * D * 2;   // K rows of one half-tile

  frag qf[2][NCD];
  frag dof[2][NCD];
  f32x16 dq[2][NCT];
  f32x16 s[2], dp[2];   // S^T, dP^T of the current half-tile
  frag vf[NCD];         // V operand of the next half-tile
  float lse2[2];        // LSE * log2(e), +inf for an empty row
  float dl[2];          // delta
  const __bf16* kb;
  const __bf16* vb;
  int kvs;
  char* kt;             // this wave's two K buffers [2][HBYTES]
  float sl2;

  // Chunk c of row r sits at chunk index c ^ swz(r): the row reads (rows
  // {0-3, 8-11} + 4k, eight lanes at a time) and the transposed reads (four
  // consecutive rows, sixteen lanes) both hit eight distinct bank groups.
  __device__ static __forceinline__ constexpr int swz(int row) { return 2 * (row & 3) + ((row >> 3) & 1); }
  __device__ static __forceinline__ int off(int row, int chunk) {
    return (row / RPI) * 1024 + (row % RPI) * (CPR * 16) + 16 * (chunk ^ swz(row));
  }

  template <class Set>
  __device__ __forceinline__ void load_v(const Set& S, int n) {
    const int lane = threadIdx.x & 63;
    const int hl = lane >> 5;
    const unsigned key = S.key_pos(n, slot_perm<KPL>(lane & 31));
    const __bf16* vrow = vb + key * (unsigned)kvs + hl * KPL;
#pragma unroll
    for (int c = 0; c < NCD; ++c) vf[c] = load_frag<__bf16>(vrow + c * KC);
  }

  template <class Set>
  __device__ __forceinline__ void dma_k(const Set& S, int n, char* dst) const {
    typedef __attribute__((address_space(3))) void* lds_ptr;
    typedef __attribute__((address_space(1))) void* glb_ptr;
    const int lane = threadIdx.x & 63;
    const int rr = lane / CPR;
    if constexpr (Set::kContiguous) {
      const __bf16* p0 = kb + (unsigned)S.key_pos(n, rr) * (unsigned)kvs;
#pragma unroll
      for (int u = 0; u < NVL; ++u) {
        const int chunk = (lane % CPR) ^ swz(u * RPI + rr);
        __builtin_amdgcn_global_load_lds((glb_ptr)(p0 + (unsigned)(u * RPI * kvs) + chunk * 8),
                                         (lds_ptr)(dst + u * 1024), 16, 0, 0);
      }
    } else {
#pragma unroll
      for (int u = 0; u < NVL; ++u) {
        const int chunk = (lane % CPR) ^ swz(u * RPI + rr);
        __builtin_amdgcn_global_load_lds(
            (glb_ptr)(kb + (unsigned)S.key_pos(n, rr + u * RPI) * (unsigned)kvs + chunk * 8),
            (lds_ptr)(dst + u * 1024), 16, 0, 0);
      }
    }
  }

  // A operand of S^T = K Q^T: key slot_perm(L%32), chunk 2c + L/32.
  __device__ __forceinline__ static frag k_row_frag(const char* src, int c) {
    const int lane = threadIdx.x & 63;
    return *reinterpret_cast<const frag*>(src + off(slot_perm<KPL>(lane & 31), 2 * c + (lane >> 5)));
  }

  // A operand of dQ^T += K^T dS^T: channels 32ct + L%32, keys of k chunk c.
  // ds_read_b64_tr_b16: in each 16-lane group, lane i receives element i%4
  // of the 8 bytes read by lanes i/4, 4+i/4, 8+i/4, 12+i/4.
  __device__ __forceinline__ static frag kt_frag(const char* src, int ct, int c) {
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4;
    const int sg = lane & 15;
    const int hl = lane >> 5;
    const int cb = 32 * ct + 16 * (g & 1) + 4 * (sg & 3);
    typedef short v4s __attribute__((ext_vector_type(4)));
    typedef short v8s __attribute__((ext_vector_type(8)));
    v4s part[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int row = c * 16 + 8 * hl + 4 * q + (sg >> 2);
      part[q] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) v4s*)(src + off(row, cb >> 3) + 2 * (cb & 7)));
    }
    const v8s both = __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(frag, both);
  }

  __device__ __forceinline__ void scores(const char* src) {
#pragma unroll
    for (int rg = 0; rg < 2; ++rg) {
      s[rg] = f32x16{0};
      dp[rg] = f32x16{0};
#pragma unroll
      for (int c = 0; c < NCD; ++c) {
        s[rg] = MF::mma(k_row_frag(src, c), qf[rg][c], s[rg]);
        dp[rg] = MF::mma(vf[c], dof[rg][c], dp[rg]);
      }
    }
  }

  template <class Set>
  __device__ __forceinline__ void dscores(const Set& S, int n, frag (&dsf)[2][NCK]) {
    const int lane = threadIdx.x & 63;
    const int hl = lane >> 5;
    const int l32 = lane & 31;
    if (!S.full(n)) {
#pragma unroll
      for (int rg = 0; rg < 2; ++rg)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (!S.valid(n, reg_row<KPL>(i, hl), 32 * rg + l32)) s[rg][i] = -INFINITY;
    }
#pragma unroll
    for (int rg = 0; rg < 2; ++rg) {
      float ds[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float pr = fast_exp2(__builtin_fmaf(s[rg][i], sl2, -lse2[rg]));
        ds[i] = pr * (dp[rg][i] - dl[rg]);
      }
#pragma unroll
      for (int c = 0; c < NCK; ++c) dsf[rg][c] = MF::pack(&ds[c * KPL]);
    }
  }

  __device__ __forceinline__ void dqmma(const char* src, const frag (&dsf)[2][NCK]) {
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int c = 0; c < NCK; ++c) {
        const frag a = kt_frag(src, ct, c);
#pragma unroll
        for (int rg = 0; rg < 2; ++rg) dq[rg][ct] = MF::mma(a, dsf[rg][c], dq[rg][ct]);
      }
  }

  template <class Set>
  __device__ __forceinline__ void step(const Set& S, int n, int N) {
    frag dsf[2][NCK];
    const int n1 = n + 1 < N ? n + 1 : N - 1;
    load_v(S, n1);
    dma_k(S, n1, kt + ((n + 1) & 1) * HBYTES);
    dscores(S, n, dsf);
    dqmma(kt + (n & 1) * HBYTES, dsf);
    __builtin_amdgcn_s_waitcnt(vmcnt_wait(0));
    wave_sync();
    scores(kt + ((n + 1) & 1) * HBYTES);
  }

  template <class Set>
  __device__ __forceinline__ void run(const Set& S) {
    const int N = S.n_halves();
    if (N == 0) return;
    dma_k(S, 0, kt);
    load_v(S, 0);
    __builtin_amdgcn_s_waitcnt(vmcnt_wait(0));
    wave_sync();
    scores(kt);
    for (int n = 0; n < N; ++n) step(S, n, N);
    wave_sync();
  }
};

template <int D>
__global__ __launch_bounds__(kQThreads) void vs_bwd_dq_bf16_kernel(AttnParams p) {
  typedef DqWorkerB<D> W;
  constexpr int KT_BYTES = 4 * 2 * W::HBYTES;
  constexpr int OB_PITCH = D + 4;
  constexpr int OB_BYTES = 64 * OB_PITCH * 4;
  constexpr int BUF = KT_BYTES > OB_BYTES ? KT_BYTES : OB_BYTES;
  __shared__ QMajorLds<> L;
  __shared__ __attribute__((aligned(16))) char buf[BUF];

  int hb, i_local;
  qmajor_item(p, blockIdx.x, &hb, &i_local);
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
  const __bf16* q = reinterpret_cast<const __bf16*>(p.q);
  const __bf16* dout = reinterpret_cast<const __bf16*>(p.dout);
  const size_t row0 = (size_t)b * p.n_q + (size_t)i_local * kBlock;
#pragma unroll
  for (int rg = 0; rg < 2; ++rg) {
    const size_t roff = ((row0 + 32 * rg + l32) * p.h_q + h) * D + hl * W::KPL;
#pragma unroll
    for (int c = 0; c < W::NCD; ++c) {
      wk.qf[rg][c] = load_frag<__bf16>(q + roff + c * W::KC);
      wk.dof[rg][c] = load_frag<__bf16>(dout + roff + c * W::KC);
    }
#pragma unroll
    for (int ct = 0; ct < W::NCT; ++ct) wk.dq[rg][ct] = f32x16{0};
    const size_t li = ((size_t)b * p.h_q + h) * p.n_q + (size_t)i_local * kBlock + 32 * rg + l32;
    const float lse = p.lse[li];
    wk.lse2[rg] = (lse == -INFINITY) ? INFINITY : lse * kLog2e;
    wk.dl[rg] = p.delta[li];
  }
  wk.kvs = p.h_kv * D;
  wk.kb = reinterpret_cast<const __bf16*>(p.k) + (size_t)b * p.n_k * wk.kvs + (size_t)kvh * D;
  wk.vb = reinterpret_cast<const __bf16*>(p.v) + (size_t)b * p.n_k * wk.kvs + (size_t)kvh * D;
  wk.kt = buf + wave * 2 * W::HBYTES;
  wk.sl2 = p.sl2;

  qmajor_drive(p, rb, list, L, wk);

  float* ob = reinterpret_cast<float*>(buf);
  for (int w = 0; w < 4; ++w) {
    if (wave == w) {
#pragma unroll
      for (int rg = 0; rg < 2; ++rg)
#pragma unroll
        for (int ct = 0; ct < W::NCT; ++ct)
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4) {
            float* dst = ob + (32 * rg + l32) * OB_PITCH + 32 * ct + 8 * i4 + 4 * hl;
            f32x4 v;
#pragma unroll
            for (int u = 0; u < 4; ++u) v[u] = wk.dq[rg][ct][4 * i4 + u];
            if (w == 0) *reinterpret_cast<f32x4*>(dst) = v;
            else *reinterpret_cast<f32x4*>(dst) = *reinterpret_cast<f32x4*>(dst) + v;
          }
    }
    __syncthreads();
  }
  for (int x = tid; x < 64 * D / 4; x += kQThreads) {
    const int r = x / (D / 4);
    const int c4 = (x % (D / 4)) * 4;
    const f32x4 v = *reinterpret_cast<const f32x4*>(ob + r * OB_PITCH + c4) * p.scale;
    float* dst = p.dq + ((row0 + r) * p.h_q + h) * D + c4;
    if (p.dq_accumulate) *reinterpret_cast<f32x4*>(dst) = *reinterpret_cast<f32x4*>(dst) + v;
    else *reinterpret_cast<f32x4*>(dst) = v;
  }
}

// Row-split dQ: a workgroup of 2*NS waves serves NS key streams, the two
// waves of a stream own rows 0-31 and 32-63 and share its K and V tiles in
// LDS (both read row-wise for S^T = K Q^T and dP^T = V dO^T, K also
// transposed for dQ^T += K^T dS^T).  Each wave holds Q^T, dO^T and dQ^T of
// its 32 rows (about 220 registers), so with NS = 2 (80 KB of LDS) two
// independent workgroups share a CU.
template <int D>
struct DqRowsWorker : RowsTiles<D> {
  typedef RowsTiles<D> T;
  typedef typename T::MF MF;
  typedef typename T::frag frag;
  using T::KPL;
  using T::NCD;
  using T::NCT;
  using T::NCK;
  using T::NVH;
  using T::kb;
  using T::vb;
  using T::rh;
  using T::k_frag;
  using T::t_frag;
  using T::dma_half;

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
    if (!S.full(n)) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (!S.valid(n, reg_row<KPL>(i, hl), r)) s[i] = -INFINITY;
    }
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
    if (n < N) {
      frag dsf[NCK];
      dscores(S, n, dsf);
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int c = 0; c < NCK; ++c) dq[ct] = MF::mma(t_frag(kt[P], ct, c), dsf[c], dq[ct]);
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_wait(0) & lgkmcnt_wait0());
    __syncthreads();
    if (n + 2 < N) {
      dma_half(S, n + 2, kb, kta[P]);
      dma_half(S, n + 2, vb, vta[P]);
    }
    if (n + 1 < N) scores(kt[P ^ 1], vt[P ^ 1]);
  }

  // All waves take the same number of steps (the longest stream's), so that
  // every barrier is reached by everyone.
  template <class Set>
  __device__ __forceinline__ void run(const Set& S) {
    const int NA = S.n_halves_max();
    if (NA == 0) return;
    const int N = S.n_halves();
    if (N > 0) {
      dma_half(S, 0, kb, kta[0]);
      dma_half(S, 0, vb, vta[0]);
      dma_half(S, 1, kb, kta[1]);
      dma_half(S, 1, vb, vta[1]);
    }
    // this wave's loads of K(0), V(0) have landed (K(1), V(1) may not have)
    __builtin_amdgcn_s_waitcnt(vmcnt_wait(2 * NVH));
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

template <int D, int NS>
__global__ __launch_bounds__(128 * NS) __attribute__((amdgpu_waves_per_eu(2))) void vs_bwd_dq_rows_kernel(AttnParams p) {
  typedef DqRowsWorker<D> W;
  constexpr int NT = 128 * NS;
  constexpr int OB_PITCH = D + 4;
  constexpr int OB_BYTES = 64 * OB_PITCH * 4;
  // [ring slot][K, V][stream] tiles
  constexpr int TILES = 2 * 2 * NS * W::TB;
  __shared__ QMajorLds<NT, kColBatch, kRowsBitWords> L;
  __shared__ __attribute__((aligned(16))) char tiles[TILES > OB_BYTES ? TILES : OB_BYTES];

  int hb, i_local;
  qmajor_item(p, blockIdx.x, &hb, &i_local);
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
  wk.rh = wave / NS;
  const int r = 32 * wk.rh + l32;  // this lane's row of the block
  const __bf16* q = reinterpret_cast<const __bf16*>(p.q);
  const __bf16* dout = reinterpret_cast<const __bf16*>(p.dout);
  const size_t row0 = (size_t)b * p.n_q + (size_t)i_local * kBlock;
  {
    const size_t roff = ((row0 + r) * p.h_q + h) * D + hl * W::KPL;
#pragma unroll
    for (int c = 0; c < W::NCD; ++c) {
      wk.qf[c] = load_frag<__bf16>(q + roff + c * W::KC);
      wk.dof[c] = load_frag<__bf16>(dout + roff + c * W::KC);
    }
    const size_t li = ((size_t)b * p.h_q + h) * p.n_q + (size_t)i_local * kBlock + r;
    const float lse = p.lse[li];
    wk.lse2 = (lse == -INFINITY) ? INFINITY : lse * kLog2e;
    wk.dl = p.delta[li];
  }
#pragma unroll
  for (int ct = 0; ct < W::NCT; ++ct) wk.dq[ct] = f32x16{0};
  wk.kvs = p.h_kv * D;
  wk.kb = reinterpret_cast<const __bf16*>(p.k) + (size_t)b * p.n_k * wk.kvs + (size_t)kvh * D;
  wk.vb = reinterpret_cast<const __bf16*>(p.v) + (size_t)b * p.n_k * wk.kvs + (size_t)kvh * D;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    wk.kt[i] = tiles + ((i * 2 + 0) * NS + ks) * W::TB;
    wk.vt[i] = tiles + ((i * 2 + 1) * NS + ks) * W::TB;
    wk.kta[i] = lds_addr(wk.kt[i]);
    wk.vta[i] = lds_addr(wk.vt[i]);
  }
  wk.sl2 = p.sl2;
  wk.init_offsets();

  qmajor_drive<NS>(p, rb, list, L, wk);

  // Sum the streams' dQ^T of every row, then scale and store (or add).
  float* ob = reinterpret_cast<float*>(tiles);
  for (int w = 0; w < NS; ++w) {
    if (ks == w) {
#pragma unroll
      for (int ct = 0; ct < W::NCT; ++ct)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          float* dst = ob + r * OB_PITCH + 32 * ct + 8 * i4 + 4 * hl;
          f32x4 v;
#pragma unroll
          for (int u = 0; u < 4; ++u) v[u] = wk.dq[ct][4 * i4 + u];
          if (w == 0) *reinterpret_cast<f32x4*>(dst) = v;
          else *reinterpret_cast<f32x4*>(dst) = *reinterpret_cast<f32x4*>(dst) + v;
        }
    }
    __syncthreads();
  }
  for (int x = tid; x < 64 * D / 4; x += NT) {
    const int rr = x / (D / 4);
    const int c4 = (x % (D / 4)) * 4;
    const f32x4 v = *reinterpret_cast<const f32x4*>(ob + rr * OB_PITCH + c4) * p.scale;
    float* dst = p.dq + ((row0 + rr) * p.h_q + h) * D + c4;
    if (p.dq_accumulate) *reinterpret_cast<f32x4*>(dst) = *reinterpret_cast<f32x4*>(dst) + v;
    else *reinterpret_cast<f32x4*>(dst) = v;
  }
}

hipError_t launch_bwd_dq_bf16(const AttnParams& p, int d, hipStream_t st) {
  const dim3 gq((unsigned)(p.batch * p.h_q * p.nqb));
  if (gq.x == 0) return hipSuccess;
  // the row-split kernel's bitmap covers segments of up to 32 * kRowsBitWords blocks
  const bool rows = max_segment_blocks(p) <= 32 * kRowsBitWords;
  if (d == 128 && rows) VS_TRACED(st, "vs_bwd_dq", hipLaunchKernelGGL((vs_bwd_dq_rows_kernel<128, 2>), gq, dim3(256), 0, st, p));
  else if (d == 64 && rows) VS_TRACED(st, "vs_bwd_dq", hipLaunchKernelGGL((vs_bwd_dq_rows_kernel<64, 2>), gq, dim3(256), 0, st, p));
  else if (d == 128) VS_TRACED(st, "vs_bwd_dq", hipLaunchKernelGGL((vs_bwd_dq_bf16_kernel<128>), gq, dim3(kQThreads), 0, st, p));
  else VS_TRACED(st, "vs_bwd_dq", hipLaunchKernelGGL((vs_bwd_dq_bf16_kernel<64>), gq, dim3(kQThreads), 0, st, p));
  return hipGetLastError();
}

}  // namespace vs
