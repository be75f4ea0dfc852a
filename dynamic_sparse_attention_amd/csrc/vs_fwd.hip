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
  static constexpr bool kBf16 = sizeof(T) == 2;
  static constexpr int KPL = MF::KPL;
  static constexpr int KC = 2 * KPL;
  static constexpr int NCD = D / KC;   // k chunks over head_dim
  static constexpr int NCT = D / 32;   // 32-channel output tiles
  static constexpr int NCK = 32 / KC;  // k chunks over 32 keys
  // bf16: the 32 V rows of a half-tile go global -> LDS directly
  // (global_load_lds_dwordx4, 1 KiB per instruction = RPI rows), with the
  // 16-byte chunks of row r stored at chunk index c ^ 2*(r % 4) so that the
  // transposed reads (ds_read_b64_tr_b16) of four consecutive rows hit
  // distinct banks.
  static constexpr int CPR = D / 8;                      // 16-byte chunks per row
  static constexpr int RPI = 64 / CPR;                   // rows per load instruction
  static constexpr int NVL = 32 / RPI;                   // V load instructions per half
  // fp32: V transposed through registers into [channel][key] (pitch VTP).
  static constexpr int VTP = 32 + 4;
  static constexpr int CG = 4;                           // fp32 channels per 16-byte load
  static constexpr int KG = 2;                           // fp32 keys per 8-byte store
  static constexpr int NKG = 32 / KG;
  static constexpr int NVG = kBf16 ? 1 : NKG * (D / CG) / 64;
  static constexpr int VBUF = kBf16 ? 32 * D * 2 : D * VTP * 4;  // bytes per staging buffer
  // Rescale the output only when a row max grows by more than 2^8 (in the
  // exp2 domain): exp2(t - m) then stays below 256, exact enough in bf16/fp32.
  static constexpr float kRescale = 8.f;

  // The half-tile in flight: K operand and S^T.
  struct Buf {
    frag k[NCD];
    f32x16 s[2];
  };

  frag qf[2][NCD];
  f32x16 o[2][NCT];
  f32x4 vr[kBf16 ? 1 : NVG * KG];   // fp32 path: raw V rows of the next half-tile
  float m[2], l[2];
  const T* kb;   // K of (batch, kv head): row pos at kb + pos * kvs
  const T* vb;
  int kvs;
  char* vt;      // this wave's two staging buffers [2][VBUF]
  float sl2;

  template <class Set>
  __device__ __forceinline__ void load_k(const Set& S, int n, Buf& B) const {
    const int lane = threadIdx.x & 63;
    const int hl = lane >> 5;
    const int l32 = lane & 31;
    // A operand of S^T = K Q^T: slot l32 loads key slot_perm(l32) of the half.
    const unsigned key = S.key_pos(n, slot_perm<KPL>(l32));
    const T* krow = kb + key * (unsigned)kvs + hl * KPL;
#pragma unroll
    for (int c = 0; c < NCD; ++c) B.k[c] = load_frag<T>(krow + c * KC);
  }

  // bf16: V rows of half n straight into staging buffer dst (asynchronous;
  // NVL vector-memory instructions).  fp32: into registers.
  template <class Set>
  __device__ __forceinline__ void load_v(const Set& S, int n, char* dst) {
    const int lane = threadIdx.x & 63;
    if constexpr (kBf16) {
      const int rr = lane / CPR;
      const int chunk = (lane % CPR) ^ (2 * (rr & 3));
      typedef __attribute__((address_space(3))) void* lds_ptr;
      typedef __attribute__((address_space(1))) void* glb_ptr;
      if constexpr (Set::kContiguous) {
        const T* p0 = vb + (unsigned)S.key_pos(n, rr) * (unsigned)kvs + chunk * 8;
#pragma unroll
        for (int u = 0; u < NVL; ++u)
          __builtin_amdgcn_global_load_lds((glb_ptr)(p0 + (unsigned)(u * RPI * kvs)),
                                           (lds_ptr)(dst + u * 1024), 16, 0, 0);
      } else {
#pragma unroll
        for (int u = 0; u < NVL; ++u)
          __builtin_amdgcn_global_load_lds(
              (glb_ptr)(vb + (unsigned)S.key_pos(n, rr + u * RPI) * (unsigned)kvs + chunk * 8),
              (lds_ptr)(dst + u * 1024), 16, 0, 0);
      }
    } else {
#pragma unroll
      for (int g = 0; g < NVG; ++g) {
        const int gi = g * 64 + lane;
        const int kg = gi % NKG;
        const int cg = gi / NKG;
#pragma unroll
        for (int u = 0; u < KG; ++u)
          vr[g * KG + u] = *reinterpret_cast<const f32x4*>(vb + (unsigned)S.key_pos(n, kg * KG + u) * (unsigned)kvs + cg * CG);
      }
    }
  }

  // fp32 path: raw V rows transposed into dst[channel][key].
  __device__ __forceinline__ void stage(char* dst) const {
    if constexpr (!kBf16) {
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
  }

  // A operand of O^T += V^T P^T: channels 32ct + L%32, keys of k chunk c.
  __device__ __forceinline__ frag vt_frag(const char* src, int ct, int c) const {
    const int lane = threadIdx.x & 63;
    if constexpr (kBf16) {
      // ds_read_b64_tr_b16: in each 16-lane group, lane i receives element
      // i%4 of the 8 bytes read by lanes i/4, 4+i/4, 8+i/4, 12+i/4.  Lane sigma
      // reads key row k0 + sigma/4, channels cb + 4*(sigma%4) .. +3, so lane i
      // gets channel cb + i of keys k0 .. k0+3 (k0 is a multiple of 4).
      const int g = lane >> 4;
      const int sg = lane & 15;
      const int hl = lane >> 5;
      const int rr = sg >> 2;                               // row within the 4-row group
      const int cb = 32 * ct + 16 * (g & 1) + 4 * (sg & 3);  // first channel read
      typedef short v4s __attribute__((ext_vector_type(4)));
      typedef short v8s __attribute__((ext_vector_type(8)));
      v4s part[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int row = c * 16 + 8 * hl + 4 * q + rr;
        const int off = (row / RPI) * 1024 + (row % RPI) * (CPR * 16) +
                        16 * ((cb >> 3) ^ (2 * (row & 3))) + 2 * (cb & 7);
        part[q] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(src + off));
      }
      const v8s both = __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7);
      return __builtin_bit_cast(frag, both);
    } else {
      const int hl = lane >> 5;
      const int l32 = lane & 31;
      return reinterpret_cast<const float*>(src)[(32 * ct + l32) * VTP + c * KC + hl * KPL];
    }
  }

  __device__ __forceinline__ void scores(Buf& B) const {
#pragma unroll
    for (int rg = 0; rg < 2; ++rg) {
      B.s[rg] = f32x16{0};
#pragma unroll
      for (int c = 0; c < NCD; ++c) B.s[rg] = MF::mma(B.k[c], qf[rg][c], B.s[rg]);
    }
  }

  // Online softmax, first part: masked row maxima of half-tile n and the
  // (rare) rescale of the running state.  Masks the scores in place.
  template <class Set>
  __device__ __forceinline__ void softmax_max(const Set& S, int n, Buf& B) {
    const int lane = threadIdx.x & 63;
    const int hl = lane >> 5;
    const int l32 = lane & 31;
    if (!S.full(n)) {
#pragma unroll
      for (int rg = 0; rg < 2; ++rg) {
        const int r = 32 * rg + l32;
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (!S.valid(n, reg_row<KPL>(i, hl), r)) B.s[rg][i] = -INFINITY;
      }
    }
    float tm[2];
#pragma unroll
    for (int rg = 0; rg < 2; ++rg) {
      float mx = B.s[rg][0];
#pragma unroll
      for (int i = 1; i < 16; ++i) mx = fmaxf(mx, B.s[rg][i]);
      mx = fmaxf(mx, xor32(mx));
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
  // P^T of both row groups as bf16 (or fp32) B operands.
  __device__ __forceinline__ void softmax_exp(const Buf& B, frag (&pf)[2][NCK]) {
#pragma unroll
    for (int rg = 0; rg < 2; ++rg) {
      const float mu = (m[rg] == -INFINITY) ? 0.f : m[rg];
      float p[16];
      float rs = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        p[i] = fast_exp2(__builtin_fmaf(B.s[rg][i], sl2, -mu));
        rs += p[i];
      }
      rs += xor32(rs);
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

  // Half-tile n with cur = its data; nxt.k holds the K operand of half n+1
  // and vr the raw V rows of half n+1 (both loaded one step earlier).  The
  // step is branch-free apart from the rare rescale, so the scheduler can
  // overlap S(n+1) on the matrix cores with the exponentials of n, and P V(n)
  // with the loads of n+2.  Past the end the last half is reloaded and
  // recomputed instead of branching (its results are unused).
  // Half-tile n: b.s holds S^T(n); staging buffer n&1 holds (or is receiving)
  // V of half n.  K(n+1) is requested first so that its latency hides behind
  // the softmax of n; V(n+1) goes to the other buffer while S^T(n+1) runs on
  // the matrix cores.  Past the end the last half is reloaded and recomputed
  // instead of branching (results unused).
  template <class Set>
  __device__ __forceinline__ void step(const Set& S, int n, int N, Buf& b) {
    frag pf[2][NCK];
    const int n1 = n + 1 < N ? n + 1 : N - 1;
    load_k(S, n1, b);
    softmax_max(S, n, b);
    softmax_exp(b, pf);
    char* cur = vt + (n & 1) * VBUF;
    char* nxt = vt + ((n + 1) & 1) * VBUF;
    if constexpr (kBf16) {
      load_v(S, n1, nxt);
      scores(b);
      // everything but the NVL loads of V(n+1) has landed: V(n) is in LDS
      __builtin_amdgcn_s_waitcnt(vmcnt_wait(NVL));
    } else {
      stage(nxt);
      load_v(S, n + 2 < N ? n + 2 : N - 1, nullptr);
      scores(b);
    }
    wave_sync();
    pv(cur, pf);
  }

  template <class Set>
  __device__ __forceinline__ void run(const Set& S) {
    const int N = S.n_halves();
    if (N == 0) return;
    Buf b;
    load_v(S, 0, vt);
    if constexpr (!kBf16) {
      stage(vt);
      load_v(S, N > 1 ? 1 : 0, nullptr);
    }
    load_k(S, 0, b);
    scores(b);
    for (int n = 0; n < N; ++n) step(S, n, N, b);
    __builtin_amdgcn_s_waitcnt(vmcnt_wait(0));
    wave_sync();
  }
};

template <typename T, int D>
struct FwdLds {
  static constexpr int VT_BYTES = 4 * 2 * FwdWorker<T, D>::VBUF;
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
  wk.vt = buf + wave * 2 * W::VBUF;
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
