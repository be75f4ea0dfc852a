// vs_fwd.hip — sparse attention forward over the Vertical-Slash support.
//
// MTraining paper note, Algorithm 1 (last step) and Algorithm 2
// (block_bar_sparse_attention_forward): O = softmax(S) V and LSE over the
// support only; online softmax with a running max, a correction factor and
// a running sum ("Ring Attention Paper Analysis", "The Blockwise
// Partitioning Strategy").
//
// gfx950 design: one workgroup (4 waves) per (batch, Q head, 64-row query
// block).  Every wave holds Q^T for all 64 rows in registers and consumes
// whole 64-key tiles on its own (split over keys, not rows), so a K or V row
// is read by exactly one wave: K goes straight from global memory into the
// A operand of S^T = K Q^T, V is transposed through the wave's own LDS
// region for the A operand of O^T += V^T P^T, and P^T feeds the second
// product from registers (slot_perm).  Softmax state is fp32; P is rounded
// to bf16 for the matrix cores when the inputs are bf16.  The four waves'
// (max, sum, O) merge through LDS at the end.
#include "vs_qmajor.h"
#include "vs_trace.h"

namespace vs {

template <typename T, int D>
struct FwdWorker {
  typedef Mfma<T> MF;
  typedef typename MF::frag frag;
  static constexpr int KPL = MF::KPL;
  static constexpr int KC = 2 * KPL;
  static constexpr int NCD = D / KC;   // k chunks over head_dim
  static constexpr int NCT = D / 32;   // 32-channel output tiles
  static constexpr int NCK = 32 / KC;  // k chunks over 32 keys
  static constexpr int VTP = 32 + 16 / (int)sizeof(T);  // V^T row pitch (elements)
  static constexpr int CG = 16 / (int)sizeof(T);        // channels per 16-byte load
  static constexpr int KG = 8 / (int)sizeof(T);         // keys per 8-byte LDS store

  frag qf[2][NCD];
  f32x16 o[2][NCT];
  float m[2], l[2];
  const T* kb;   // K of (batch, kv head): row pos at kb + pos * kvs
  const T* vb;
  int kvs;
  T* vt;         // this wave's V^T staging area [D][VTP]
  float sl2;

  template <class Tile>
  __device__ __forceinline__ void half(const Tile& t, int kk) {
    const int lane = threadIdx.x & 63;
    const int hl = lane >> 5;
    const int l32 = lane & 31;
    // A operand of S^T = K Q^T: slot l32 loads key slot_perm(l32) of this half.
    const T* krow = kb + (size_t)t.key_pos(32 * kk + slot_perm<KPL>(l32)) * kvs;
    frag kf[NCD];
#pragma unroll
    for (int c = 0; c < NCD; ++c) kf[c] = load_frag<T>(krow + c * KC + hl * KPL);
    // V rows of this half, transposed into vt[channel][key].
    constexpr int NKG = 32 / KG;
    constexpr int NGRP = NKG * (D / CG);
#pragma unroll
    for (int g0 = 0; g0 < NGRP; g0 += 64) {
      const int g = g0 + lane;
      const int kg = g % NKG;
      const int cg = g / NKG;
      T vals[KG][CG];
#pragma unroll
      for (int u = 0; u < KG; ++u) {
        const T* vrow = vb + (size_t)t.key_pos(32 * kk + kg * KG + u) * kvs + cg * CG;
        *reinterpret_cast<f32x4*>(&vals[u][0]) = *reinterpret_cast<const f32x4*>(vrow);
      }
#pragma unroll
      for (int c = 0; c < CG; ++c) {
        T pk[KG];
#pragma unroll
        for (int u = 0; u < KG; ++u) pk[u] = vals[u][c];
        *reinterpret_cast<f32x2*>(vt + (cg * CG + c) * VTP + kg * KG) =
            *reinterpret_cast<const f32x2*>(pk);
      }
    }
    f32x16 s[2];
#pragma unroll
    for (int rg = 0; rg < 2; ++rg) {
      s[rg] = f32x16{0};
#pragma unroll
      for (int c = 0; c < NCD; ++c) s[rg] = MF::mma(kf[c], qf[rg][c], s[rg]);
    }
    frag pf[2][NCK];
#pragma unroll
    for (int rg = 0; rg < 2; ++rg) {
      const int r = 32 * rg + l32;
      float tt[16];
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int e = 32 * kk + reg_row<KPL>(i, hl);
        tt[i] = t.valid(e, r) ? s[rg][i] * sl2 : -INFINITY;
        mx = fmaxf(mx, tt[i]);
      }
      mx = fmaxf(mx, xor32(mx));
      const float m_new = fmaxf(m[rg], mx);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = fast_exp2(m[rg] - m_use);
      float rs = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        tt[i] = fast_exp2(tt[i] - m_use);
        rs += tt[i];
      }
      rs += xor32(rs);
      l[rg] = l[rg] * alpha + rs;
      m[rg] = m_new;
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) o[rg][ct] *= alpha;
#pragma unroll
      for (int c = 0; c < NCK; ++c) pf[rg][c] = MF::pack(&tt[c * KPL]);
    }
    wave_sync();
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
#pragma unroll
      for (int c = 0; c < NCK; ++c) {
        const frag vf = load_frag<T>(vt + (32 * ct + l32) * VTP + c * KC + hl * KPL);
#pragma unroll
        for (int rg = 0; rg < 2; ++rg) o[rg][ct] = MF::mma(vf, pf[rg][c], o[rg][ct]);
      }
    }
    wave_sync();
  }

  template <class Tile>
  __device__ __forceinline__ void tile(const Tile& t) {
    half(t, 0);
    half(t, 1);
  }
};

template <typename T, int D>
struct FwdLds {
  static constexpr int VTP = FwdWorker<T, D>::VTP;
  static constexpr int VT_BYTES = 4 * D * VTP * (int)sizeof(T);
  static constexpr int OB_PITCH = D + 4;
  static constexpr int OB_BYTES = 64 * OB_PITCH * 4;
  static constexpr int BUF = VT_BYTES > OB_BYTES ? VT_BYTES : OB_BYTES;
};

template <typename T, int D>
__global__ __launch_bounds__(kQThreads) void vs_fwd_kernel(AttnParams p) {
  typedef FwdWorker<T, D> W;
  typedef FwdLds<T, D> LD;
  __shared__ QMajorLds L;
  __shared__ __attribute__((aligned(16))) char buf[LD::BUF];
  __shared__ float s_m[4][64];
  __shared__ float s_l[4][64];

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
  const T* q = reinterpret_cast<const T*>(p.q);
  const size_t qrow0 = (size_t)b * p.n_q + (size_t)i_local * kBlock;
#pragma unroll
  for (int rg = 0; rg < 2; ++rg) {
    const T* qr = q + ((qrow0 + 32 * rg + l32) * p.h_q + h) * D;
#pragma unroll
    for (int c = 0; c < W::NCD; ++c) wk.qf[rg][c] = load_frag<T>(qr + c * W::KC + hl * W::KPL);
#pragma unroll
    for (int ct = 0; ct < W::NCT; ++ct) wk.o[rg][ct] = f32x16{0};
    wk.m[rg] = -INFINITY;
    wk.l[rg] = 0.f;
  }
  wk.kvs = p.h_kv * D;
  wk.kb = reinterpret_cast<const T*>(p.k) + (size_t)b * p.n_k * wk.kvs + (size_t)kvh * D;
  wk.vb = reinterpret_cast<const T*>(p.v) + (size_t)b * p.n_k * wk.kvs + (size_t)kvh * D;
  wk.vt = reinterpret_cast<T*>(buf) + wave * D * W::VTP;
  wk.sl2 = p.sl2;

  qmajor_drive(p, rb, list, L, wk);

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
            float* dst = ob + (32 * rg + l32) * LD::OB_PITCH + ch;
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
  // Normalise and write O (row-major, coalesced) and LSE.
  __shared__ float s_inv[64];
  if (tid < 64) {
    float mg = -INFINITY;
    for (int w = 0; w < 4; ++w) mg = fmaxf(mg, s_m[w][tid]);
    const float mu = (mg == -INFINITY) ? 0.f : mg;
    float lg = 0.f;
    for (int w = 0; w < 4; ++w) lg += s_l[w][tid] * fast_exp2(s_m[w][tid] - mu);
    s_inv[tid] = lg > 0.f ? 1.f / lg : 0.f;
    const float lse = lg > 0.f ? (mg + __log2f(lg)) * kLn2 : -INFINITY;
    p.lse[((size_t)b * p.h_q + h) * p.n_q + (size_t)i_local * kBlock + tid] = lse;
  }
  __syncthreads();
  for (int x = tid; x < 64 * D / 4; x += kQThreads) {
    const int r = x / (D / 4);
    const int c4 = (x % (D / 4)) * 4;
    f32x4 v = *reinterpret_cast<const f32x4*>(ob + r * LD::OB_PITCH + c4) * s_inv[r];
    const size_t off = ((qrow0 + r) * p.h_q + h) * D + c4;
    if (p.o_f32) {
      *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(p.o_out) + off) = v;
    } else if (sizeof(T) == 2) {
      bf16x4 w4;
#pragma unroll
      for (int u = 0; u < 4; ++u) w4[u] = (__bf16)v[u];
      *reinterpret_cast<bf16x4*>(reinterpret_cast<__bf16*>(p.o_out) + off) = w4;
    } else {
      *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(p.o_out) + off) = v;
    }
  }
}

hipError_t launch_fwd(const AttnParams& p, int dtype_bf16, int d, hipStream_t st) {
  const dim3 grid((unsigned)(p.batch * p.h_q * p.nqb));
  if (grid.x == 0) return hipSuccess;
  if (dtype_bf16 && d == 128) VS_TRACED(st, "vs_fwd", hipLaunchKernelGGL((vs_fwd_kernel<__bf16, 128>), grid, dim3(kQThreads), 0, st, p));
  else if (dtype_bf16 && d == 64) VS_TRACED(st, "vs_fwd", hipLaunchKernelGGL((vs_fwd_kernel<__bf16, 64>), grid, dim3(kQThreads), 0, st, p));
  else if (!dtype_bf16 && d == 128) VS_TRACED(st, "vs_fwd", hipLaunchKernelGGL((vs_fwd_kernel<float, 128>), grid, dim3(kQThreads), 0, st, p));
  else VS_TRACED(st, "vs_fwd", hipLaunchKernelGGL((vs_fwd_kernel<float, 64>), grid, dim3(kQThreads), 0, st, p));
  return hipGetLastError();
}

}  // namespace vs
