// vs_bwd.hip — sparse attention backward over the Vertical-Slash support.
//
// MTraining §3.2 Eq. 1-2 and the paper note's Appendix B.1:
//   P = exp(S - LSE), dP = dO V^T, dS = P * (dP - delta),
//   dQ = scale dS K, dK = scale dS^T Q, dV = P^T dO,
// with P recomputed from the final LSE ("Ring Attention Paper Analysis",
// "Backward Pass and Gradient Computation" and "Checkpointing Strategy"),
// over the same support as the forward pass (the backward inherits the
// forward's sparsity, MTraining §3.2).
//
// gfx950 design: three kernels, none of which needs atomics on the dense part.
//   * dQ (query-major): same walk and wave split as the forward; per 32
//     keys S^T = K Q^T and dP^T = V dO^T from registers, dQ^T += K^T dS^T with
//     K^T staged through the wave's LDS region.
//   * dK/dV over slash tiles (key-major): one workgroup per (batch, KV head,
//     key block), two waves of 32 keys each; it visits every (Q head of the
//     group, block-diagonal g) pair that reads the block, so dK and dV of the
//     block are complete in registers and are stored once.
//   * dK/dV over column tiles: one workgroup per (list, 64 gathered columns,
//     range of query blocks), added to dK/dV with fp32 atomics after the
//     slash kernel has stored its blocks (stream order).
#include "vs_qmajor.h"
#include "vs_stage.h"
#include "vs_trace.h"

namespace vs {

// ---------------------------------------------------------------------------
// dQ, query-major.
template <typename T, int D>
struct DqWorker {
  typedef Mfma<T> MF;
  typedef typename MF::frag frag;
  static constexpr int KPL = MF::KPL;
  static constexpr int KC = 2 * KPL;
  static constexpr int NCD = D / KC;
  static constexpr int NCT = D / 32;
  static constexpr int NCK = 32 / KC;
  static constexpr int KTP = 32 + 16 / (int)sizeof(T);  // K^T row pitch (elements)

  frag qf[2][NCD];
  frag dof[2][NCD];
  f32x16 dq[2][NCT];
  float lse2[2];   // LSE * log2(e), +inf for an empty row
  float dl[2];     // delta
  const T* kb;
  const T* vb;
  int kvs, vvs;    // K and V row strides (elements)
  T* kt;           // this wave's K^T staging area [D][KTP]
  float sl2;

  template <class Set>
  __device__ __forceinline__ void half(const Set& S, int n) {
    const int lane = threadIdx.x & 63;
    const int hl = lane >> 5;
    const int l32 = lane & 31;
    const int kpos = S.key_pos(n, slot_perm<KPL>(l32));
    const T* krow = kb + (size_t)kpos * kvs;
    const T* vrow = vb + (size_t)kpos * vvs;
    frag kf[NCD], vf[NCD];
#pragma unroll
    for (int c = 0; c < NCD; ++c) {
      kf[c] = load_frag<T>(krow + c * KC + hl * KPL);
      vf[c] = load_frag<T>(vrow + c * KC + hl * KPL);
    }
    stage_transposed<T, D, 32, KTP, 64>(kt, kb, [&](int r) { return (size_t)S.key_pos(n, r) * kvs; },
                                        lane);
    f32x16 s[2], dp[2];
#pragma unroll
    for (int rg = 0; rg < 2; ++rg) {
      s[rg] = f32x16{0};
      dp[rg] = f32x16{0};
#pragma unroll
      for (int c = 0; c < NCD; ++c) {
        s[rg] = MF::mma(kf[c], qf[rg][c], s[rg]);
        dp[rg] = MF::mma(vf[c], dof[rg][c], dp[rg]);
      }
    }
    const bool full = S.full(n);
    frag dsf[2][NCK];
#pragma unroll
    for (int rg = 0; rg < 2; ++rg) {
      const int r = 32 * rg + l32;
      float ds[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const bool ok = full || S.valid(n, reg_row<KPL>(i, hl), r);
        const float pr = ok ? fast_exp2(__builtin_fmaf(s[rg][i], sl2, -lse2[rg])) : 0.f;
        ds[i] = pr * (dp[rg][i] - dl[rg]);
      }
#pragma unroll
      for (int c = 0; c < NCK; ++c) dsf[rg][c] = MF::pack(&ds[c * KPL]);
    }
    wave_sync();
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
#pragma unroll
      for (int c = 0; c < NCK; ++c) {
        const frag kt_f = load_frag<T>(kt + (32 * ct + l32) * KTP + c * KC + hl * KPL);
#pragma unroll
        for (int rg = 0; rg < 2; ++rg) dq[rg][ct] = MF::mma(kt_f, dsf[rg][c], dq[rg][ct]);
      }
    }
    wave_sync();
  }

  template <class Set>
  __device__ __forceinline__ void run(const Set& S) {
    const int N = S.n_halves();
    for (int n = 0; n < N; ++n) half(S, n);
  }
};

template <typename T, int D>
__global__ __launch_bounds__(kQThreads) void vs_bwd_dq_kernel(AttnParams p) {
  typedef DqWorker<T, D> W;
  constexpr int KT_BYTES = 4 * D * W::KTP * (int)sizeof(T);
  constexpr int OB_PITCH = D + 4;
  constexpr int OB_BYTES = 64 * OB_PITCH * 4;
  constexpr int BUF = KT_BYTES > OB_BYTES ? KT_BYTES : OB_BYTES;
  __shared__ QMajorLds<> L;
  __shared__ __attribute__((aligned(16))) char buf[BUF];

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
  const T* q = reinterpret_cast<const T*>(p.q);
  const T* dout = reinterpret_cast<const T*>(p.dout);
  const int row0 = i_local * kBlock;  // first row of the block in this batch row
#pragma unroll
  for (int rg = 0; rg < 2; ++rg) {
    const size_t qoff = p.sq.at(b, row0 + 32 * rg + l32, h);
    const size_t doff = p.sdo.at(b, row0 + 32 * rg + l32, h);
#pragma unroll
    for (int c = 0; c < W::NCD; ++c) {
      wk.qf[rg][c] = load_frag<T>(q + qoff + c * W::KC + hl * W::KPL);
      wk.dof[rg][c] = load_frag<T>(dout + doff + c * W::KC + hl * W::KPL);
    }
#pragma unroll
    for (int ct = 0; ct < W::NCT; ++ct) wk.dq[rg][ct] = f32x16{0};
    const size_t li = ((size_t)b * p.h_q + h) * p.n_q + (size_t)i_local * kBlock + 32 * rg + l32;
    const float lse = p.lse[li];
    wk.lse2[rg] = (lse == -INFINITY) ? INFINITY : lse * kLog2e;
    wk.dl[rg] = p.delta[li];
  }
  wk.kvs = (int)p.sk.t;
  wk.vvs = (int)p.sv.t;
  wk.kb = reinterpret_cast<const T*>(p.k) + p.sk.at(b, 0, kvh);
  wk.vb = reinterpret_cast<const T*>(p.v) + p.sv.at(b, 0, kvh);
  wk.kt = reinterpret_cast<T*>(buf) + wave * D * W::KTP;
  wk.sl2 = p.sl2;

  qmajor_drive(p, rb, list, L, qm_bits, wk);

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
    float* dst = p.dq + (((size_t)b * p.n_q + row0 + r) * p.h_q + h) * D + c4;
    if (p.dq_accumulate) *reinterpret_cast<f32x4*>(dst) = *reinterpret_cast<f32x4*>(dst) + v;
    else *reinterpret_cast<f32x4*>(dst) = v;
  }
}

// ---------------------------------------------------------------------------
// dK / dV, key-major.  Two waves; wave kh owns keys 32*kh .. 32*kh+31 of a
// 64-key unit and accumulates dK^T, dV^T for them over all query tiles.
constexpr int kKThreads = 128;

template <typename T, int D>
struct KvWorker {
  typedef Mfma<T> MF;
  typedef typename MF::frag frag;
  static constexpr int KPL = MF::KPL;
  static constexpr int KC = 2 * KPL;
  static constexpr int NCD = D / KC;
  static constexpr int NCT = D / 32;
  static constexpr int NCK = 32 / KC;
  static constexpr int NCR = 64 / KC;                     // k chunks over 64 rows
  static constexpr int RTP = 64 + 16 / (int)sizeof(T);    // Q^T / dO^T row pitch (elements)

  frag kB[NCD];     // B operand K^T for this wave's keys
  frag vB[NCD];     // B operand V^T
  f32x16 dk[NCT];   // dK^T [channel][key]
  f32x16 dv[NCT];   // dV^T [channel][key]

  // One query tile of 64 rows (LDS: Q^T, dO^T, lse2, delta already staged).
  // valid(r) for this lane's key column and row r.
  template <class ValidF>
  __device__ __forceinline__ void tile(const T* qrows, const T* dorows, size_t qstride, size_t dostride,
                                       const T* qt, const T* dot, const float* s_lse2, const float* s_del,
                                       float sl2, ValidF valid) {
    const int lane = threadIdx.x & 63;
    const int hl = lane >> 5;
    const int l32 = lane & 31;
    f32x16 s[2], dp[2];
#pragma unroll
    for (int rg = 0; rg < 2; ++rg) {
      const size_t rr = (size_t)(32 * rg + slot_perm<KPL>(l32));
      s[rg] = f32x16{0};
      dp[rg] = f32x16{0};
#pragma unroll
      for (int c = 0; c < NCD; ++c) {
        const frag qa = load_frag<T>(qrows + rr * qstride + c * KC + hl * KPL);
        const frag da = load_frag<T>(dorows + rr * dostride + c * KC + hl * KPL);
        s[rg] = MF::mma(qa, kB[c], s[rg]);
        dp[rg] = MF::mma(da, vB[c], dp[rg]);
      }
    }
    frag pf[2][NCK], dsf[2][NCK];
#pragma unroll
    for (int rg = 0; rg < 2; ++rg) {
      float pr[16], ds[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = 32 * rg + reg_row<KPL>(i, hl);
        const float x = valid(r) ? fast_exp2(s[rg][i] * sl2 - s_lse2[r]) : 0.f;
        pr[i] = x;
        ds[i] = x * (dp[rg][i] - s_del[r]);
      }
#pragma unroll
      for (int c = 0; c < NCK; ++c) {
        pf[rg][c] = MF::pack(&pr[c * KPL]);
        dsf[rg][c] = MF::pack(&ds[c * KPL]);
      }
    }
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
#pragma unroll
      for (int c = 0; c < NCR; ++c) {
        const int rg = c / NCK;
        const int cc = c % NCK;
        const frag doa = load_frag<T>(dot + (32 * ct + l32) * RTP + c * KC + hl * KPL);
        const frag qa = load_frag<T>(qt + (32 * ct + l32) * RTP + c * KC + hl * KPL);
        dv[ct] = MF::mma(doa, pf[rg][cc], dv[ct]);
        dk[ct] = MF::mma(qa, dsf[rg][cc], dk[ct]);
      }
    }
  }
};

template <typename T, int D>
struct KvLds {
  static constexpr int RTP = KvWorker<T, D>::RTP;
  T qt[D * RTP];
  T dot[D * RTP];
  float lse2[64];
  float del[64];
  int tiles[kKThreads];
  int wsum[2];
};

// Stage Q^T, dO^T, LSE (log2 domain) and delta of local query block i, head h.
template <typename T, int D>
__device__ __forceinline__ void kv_stage(const AttnParams& p, KvLds<T, D>& L, int b, int h, int i) {
  const int tid = threadIdx.x;
  const T* qb = reinterpret_cast<const T*>(p.q) + p.sq.at(b, i * kBlock, h);
  const T* db = reinterpret_cast<const T*>(p.dout) + p.sdo.at(b, i * kBlock, h);
  stage_transposed<T, D, 64, KvWorker<T, D>::RTP, kKThreads>(L.qt, qb, [&](int r) { return (size_t)r * p.sq.t; }, tid);
  stage_transposed<T, D, 64, KvWorker<T, D>::RTP, kKThreads>(L.dot, db, [&](int r) { return (size_t)r * p.sdo.t; }, tid);
  const size_t li = ((size_t)b * p.h_q + h) * p.n_q + (size_t)i * kBlock;
  if (tid < 64) {
    const float lse = p.lse[li + tid];
    L.lse2[tid] = (lse == -INFINITY) ? INFINITY : lse * kLog2e;
  } else {
    L.del[tid - 64] = p.delta[li + tid - 64];
  }
}

template <typename T, int D>
__device__ __forceinline__ void kv_load_keys(KvWorker<T, D>& wk, const AttnParams& p, int b, int kvh,
                                             int kpos) {
  typedef KvWorker<T, D> W;
  const int lane = threadIdx.x & 63;
  const int hl = lane >> 5;
  const T* kr = reinterpret_cast<const T*>(p.k) + p.sk.at(b, kpos, kvh);
  const T* vr = reinterpret_cast<const T*>(p.v) + p.sv.at(b, kpos, kvh);
#pragma unroll
  for (int c = 0; c < W::NCD; ++c) {
    wk.kB[c] = load_frag<T>(kr + c * W::KC + hl * W::KPL);
    wk.vB[c] = load_frag<T>(vr + c * W::KC + hl * W::KPL);
  }
#pragma unroll
  for (int ct = 0; ct < W::NCT; ++ct) {
    wk.dk[ct] = f32x16{0};
    wk.dv[ct] = f32x16{0};
  }
}

// Write (or add) scale*dK^T and dV^T of this lane's key column.
template <typename T, int D>
__device__ __forceinline__ void kv_store(const KvWorker<T, D>& wk, const AttnParams& p, int b, int kvh,
                                         int kpos, bool atomic) {
  typedef KvWorker<T, D> W;
  const int lane = threadIdx.x & 63;
  const int hl = lane >> 5;
  const size_t off = (((size_t)b * p.n_k + kpos) * p.h_kv + kvh) * D;
#pragma unroll
  for (int ct = 0; ct < W::NCT; ++ct)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int ch = 32 * ct + 8 * i4 + 4 * hl;
      f32x4 a, v;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        a[u] = wk.dk[ct][4 * i4 + u] * p.scale;
        v[u] = wk.dv[ct][4 * i4 + u];
      }
      if (atomic) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          atomicAdd(p.dk + off + ch + u, a[u]);
          atomicAdd(p.dv + off + ch + u, v[u]);
        }
      } else {
        *reinterpret_cast<f32x4*>(p.dk + off + ch) = a;
        *reinterpret_cast<f32x4*>(p.dv + off + ch) = v;
      }
    }
}

template <typename T, int D>
__global__ __launch_bounds__(kKThreads) void vs_bwd_dkdv_slash_kernel(AttnParams p) {
  typedef KvWorker<T, D> W;
  __shared__ KvLds<T, D> L;
  const int tid = threadIdx.x;
  const int kh = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  // Work item: (batch, kv head, local key block), first key blocks first.
  const int BH = p.batch * p.h_kv;
  const int bh = blockIdx.x % BH;
  const int j = blockIdx.x / BH;
  const int b = bh / p.h_kv;
  const int kvh = bh % p.h_kv;
  const int G = p.h_q / p.h_kv;
  int kb_glob, seg, a_blk, nb_seg;
  if (p.W == 1) {
    kb_glob = j;
    seg = seg_of_block(p.seg, j);
    a_blk = p.seg.start_blk[seg];
    nb_seg = p.seg.start_blk[seg + 1] - a_blk;
  } else {
    kb_glob = global_key_block(p, j);
    seg = 0;
    a_blk = 0;
    nb_seg = p.n_global / kBlock;
  }
  const int beta_k = kb_glob - a_blk;
  const int kpos = j * kBlock + 32 * kh + l32;  // this lane's key column
  const int kin = 32 * kh + l32;                // column inside the block

  W wk;
  kv_load_keys<T, D>(wk, p, b, kvh, kpos);
  for (int hh = 0; hh < G; ++hh) {
    const int h = kvh * G + hh;
    const int list = (b * p.h_q + h) * p.seg.n_seg + seg;
    const int sp0 = p.s_ptr[list];
    const int ns = p.s_ptr[list + 1] - sp0;
    for (int base = 0; base < ns; base += kKThreads) {
      const int e = base + tid;
      int i = -1, diag = 0;
      if (e < ns) {
        const int g = p.s_idx[sp0 + e];
        if (g >= 0 && beta_k + g < nb_seg) {
          i = local_query_block(p, kb_glob + g);
          diag = g == 0;
        }
      }
      int tot;
      const int slot = block_compact<kKThreads>(i >= 0, L.wsum, &tot);
      if (i >= 0) L.tiles[slot] = 2 * i + diag;
      __syncthreads();
      for (int t = 0; t < tot; ++t) {
        const int v = L.tiles[t];
        const int qi = v >> 1;
        const bool dg = (v & 1) != 0;
        kv_stage<T, D>(p, L, b, h, qi);
        __syncthreads();
        const T* qrows = reinterpret_cast<const T*>(p.q) + p.sq.at(b, qi * kBlock, h);
        const T* drows = reinterpret_cast<const T*>(p.dout) + p.sdo.at(b, qi * kBlock, h);
        wk.tile(qrows, drows, p.sq.t, p.sdo.t, L.qt, L.dot, L.lse2, L.del, p.sl2,
                [&](int r) { return !dg || kin <= r; });
        __syncthreads();
      }
    }
  }
  kv_store<T, D>(wk, p, b, kvh, kpos, false);
}

// Column tiles: unit = (list, column tile, query-block range).
template <typename T, int D>
__global__ __launch_bounds__(kKThreads) void vs_bwd_dkdv_cols_kernel(AttnParams p) {
  typedef KvWorker<T, D> W;
  __shared__ KvLds<T, D> L;
  uint32_t* bits = qm_bits;  // (nb_seg + 31) / 32 words of dynamic LDS
  const int tid = threadIdx.x;
  const int kh = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  int u = blockIdx.x;
  const int qr = u % p.qranges;
  u /= p.qranges;
  const int ctile = u % p.col_tiles;
  const int list = u / p.col_tiles;
  const int vc = p.vcnt[list];
  if (64 * ctile >= vc) return;
  const int seg = list % p.seg.n_seg;
  const int bh = list / p.seg.n_seg;
  const int b = bh / p.h_q;
  const int h = bh % p.h_q;
  const int kvh = h * p.h_kv / p.h_q;
  int a_blk, nb_seg, i_lo, i_hi;
  if (p.W == 1) {
    a_blk = p.seg.start_blk[seg];
    nb_seg = p.seg.start_blk[seg + 1] - a_blk;
    i_lo = a_blk;
    i_hi = a_blk + nb_seg;
  } else {
    a_blk = 0;
    nb_seg = p.n_global / kBlock;
    i_lo = 0;
    i_hi = p.nqb;
  }
  const int r_lo = max(i_lo, qr * p.qrange_len);
  const int r_hi = min(i_hi, (qr + 1) * p.qrange_len);
  const int* vs = p.vsel + (size_t)list * p.vsel_stride + 64 * ctile;
  const int ncol = min(64, vc - 64 * ctile);
  // Skip ranges that end before the first column's block.
  const int first_blk = vs[0] / kBlock;
  auto qglob = [&](int i) { return p.W == 1 ? i : p.q_rank + p.W * i; };
  if (r_lo >= r_hi || qglob(r_hi - 1) < first_blk) return;

  const int col = 32 * kh + l32;
  const bool col_ok = col < ncol;
  const int m = vs[col_ok ? col : 0];
  const int bm = m / kBlock - a_blk;
  const int kpos = local_key_pos(p, m);

  const int sp0 = p.s_ptr[list];
  const int ns = p.s_ptr[list + 1] - sp0;
  const int nwords = (nb_seg + 31) >> 5;
  for (int w = tid; w < nwords; w += kKThreads) bits[w] = 0u;
  __syncthreads();
  for (int e = tid; e < ns; e += kKThreads) {
    const int g = p.s_idx[sp0 + e];
    if (g >= 0 && g < nb_seg) atomicOr(&bits[g >> 5], 1u << (g & 31));
  }
  __syncthreads();

  W wk;
  kv_load_keys<T, D>(wk, p, b, kvh, kpos);
  for (int i = r_lo; i < r_hi; ++i) {
    const int qbg = qglob(i);
    if (qbg < first_blk) continue;  // uniform across the workgroup
    const int beta_q = qbg - a_blk;
    const int off = beta_q - bm;
    const bool lane_ok = col_ok && off >= 0 && ((bits[off >> 5] >> (off & 31)) & 1u) == 0u;
    kv_stage<T, D>(p, L, b, h, i);
    __syncthreads();
    const T* qrows = reinterpret_cast<const T*>(p.q) + p.sq.at(b, i * kBlock, h);
    const T* drows = reinterpret_cast<const T*>(p.dout) + p.sdo.at(b, i * kBlock, h);
    const int row0 = qbg * kBlock;
    wk.tile(qrows, drows, p.sq.t, p.sdo.t, L.qt, L.dot, L.lse2, L.del, p.sl2,
            [&](int r) { return lane_ok && m <= row0 + r; });
    __syncthreads();
  }
  if (col_ok) kv_store<T, D>(wk, p, b, kvh, kpos, true);
}

hipError_t launch_bwd_kv_bf16(const AttnParams& p, int d, hipStream_t st);
hipError_t launch_bwd_dq_bf16(const AttnParams& p, int d, hipStream_t st);

// bf16 inputs take the direct-load kernels (vs_bwd_kv.hip, vs_bwd_dq.hip);
// fp32 inputs the kernels of this file.
hipError_t launch_bwd(const AttnParams& p, int dtype_bf16, int d, hipStream_t st) {
  if (dtype_bf16) {
    // dQ first: with delta_out / lse2_out set it writes the row terms the
    // dK/dV kernels read.
    hipError_t e = launch_bwd_dq_bf16(p, d, st);
    if (e != hipSuccess) return e;
    return launch_bwd_kv_bf16(p, d, st);
  }
  const dim3 gq((unsigned)(p.batch * p.h_q * p.nqb));
  const dim3 gs((unsigned)(p.batch * p.h_kv * p.nkb));
  const dim3 gc((unsigned)(p.batch * p.h_q * p.seg.n_seg * p.col_tiles * p.qranges));
  const size_t dyn = qmajor_bits_bytes(p);
#define VS_BWD(T, DD)                                                                           \
  do {                                                                                          \
    if (gs.x) VS_TRACED(st, "vs_bwd_dkdv_slash", hipLaunchKernelGGL((vs_bwd_dkdv_slash_kernel<T, DD>), gs, dim3(kKThreads), 0, st, p)); \
    if (gc.x) VS_TRACED(st, "vs_bwd_dkdv_cols", hipLaunchKernelGGL((vs_bwd_dkdv_cols_kernel<T, DD>), gc, dim3(kKThreads), dyn, st, p)); \
    if (gq.x) VS_TRACED(st, "vs_bwd_dq", hipLaunchKernelGGL((vs_bwd_dq_kernel<T, DD>), gq, dim3(kQThreads), dyn, st, p));               \
  } while (0)
  if (d == 128) VS_BWD(float, 128);
  else VS_BWD(float, 64);
#undef VS_BWD
  return hipGetLastError();
}

}  // namespace vs
