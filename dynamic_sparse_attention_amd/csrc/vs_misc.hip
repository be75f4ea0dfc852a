// vs_misc.hip — memory-bound helper kernels: vertical-list preparation,
// the backward row term delta, and the LSE merge of chunk partials.
#include <algorithm>

#include "vs_attn_common.h"
#include "vs_trace.h"

namespace vs {

// convert_index for verticals (MTraining paper note, Algorithm 2): keep the
// selected columns of list l that this call holds (inside the list's segment;
// for a block-striped call, in a key block of rank k_rank), in ascending
// order, as global positions.  One workgroup per list, ordered compaction
// in rounds of kPrepThreads entries.
constexpr int kPrepThreads = 1024;

__global__ __launch_bounds__(kPrepThreads) void vs_prep_vertical_kernel(AttnParams p, const int* v_ptr,
                                                                        const int* v_idx) {
  __shared__ int wsum[kPrepThreads / 64];
  const int l = blockIdx.x;
  const int s = l % p.seg.n_seg;
  int a, e;
  if (p.W == 1) {
    a = p.seg.start_blk[s] * kBlock;
    e = p.seg.start_blk[s + 1] * kBlock;
  } else {
    a = 0;
    e = p.n_global;
  }
  // the group-share accumulators (vs_group_share_kernel, which runs next)
  if (p.map_group && l == 0 && threadIdx.x < 5) p.map_group[2 + threadIdx.x] = 0;
  const int v0 = v_ptr[l];
  const int nv = v_ptr[l + 1] - v0;
  int* out = const_cast<int*>(p.vsel) + (size_t)l * p.vsel_stride;
  int count = 0;
  for (int base = 0; base < nv; base += kPrepThreads) {
    const int i = base + threadIdx.x;
    int m = -1;
    bool keep = false;
    if (i < nv) {
      m = v_idx[v0 + i];
      keep = m >= a && m < e && local_key_block(p, m / kBlock) >= 0;
    }
    int tot;
    const int slot = block_compact<kPrepThreads>(keep, wsum, &tot);
    if (keep && count + slot < p.vsel_stride) out[count + slot] = m;
    count += tot;
    __syncthreads();
  }
  if (threadIdx.x == 0) const_cast<int*>(p.vcnt)[l] = count < p.vsel_stride ? count : p.vsel_stride;
}

// Whether the Q heads of each (batch, KV head) group share their selected
// block-diagonals: over up to 1024 evenly spread lists of non-leading heads,
// the entries that the group's first head (same batch and segment) also
// selected, as a fraction of the shorter of the two lists (the first
// kShareCap entries of each, a sample for longer ones).  Measured against
// the shorter list, heads whose top-k lists are nested (budgets that differ
// per head) count as sharing, as their diagonal tiles are shared.
// share[0] = 1 when the fraction is at least one half; this picks the work
// mapping of the query-major kernels (qmajor_item).  Each wave takes one
// sampled list: it stages the leading head's list in LDS and its lanes
// binary-search their own entries in it.  Lists are ascending, with -1
// padding at the end (ordered as +inf).  The workgroups add their counts
// into share[2..5] (two 64-bit sums, zeroed by vs_prep_vertical_kernel just
// before) and take a ticket in share[6]; the last one decides.
constexpr int kShareCap = 2048;
constexpr int kShareSample = 1024;

__global__ __launch_bounds__(256) void vs_group_share_kernel(AttnParams p, int* share) {
  __shared__ int lead[4][kShareCap];
  __shared__ long long red[2][4];
  __shared__ bool last;
  const int GS = p.h_q / p.h_kv;
  const int n_lists = p.batch * p.h_q * p.seg.n_seg;
  const int stride = n_lists > kShareSample ? n_lists / kShareSample : 1;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  long long common = 0, total = 0;
  const int t = 4 * blockIdx.x + wave;  // sampled list t * stride
  if (t * stride < n_lists && t < kShareSample) {  // wave-uniform
    const int l = t * stride;
    const int seg = l % p.seg.n_seg;
    const int bh = l / p.seg.n_seg;
    const int h = bh % p.h_q;
    const int b = bh / p.h_q;
    const int h0 = (h / GS) * GS;
    if (h != h0) {
      const int l0 = (b * p.h_q + h0) * p.seg.n_seg + seg;
      const int* A = p.s_idx + p.s_ptr[l];
      const int* B = p.s_idx + p.s_ptr[l0];
      const int na = min(p.s_ptr[l + 1] - p.s_ptr[l], kShareCap);
      const int nb = min(p.s_ptr[l0 + 1] - p.s_ptr[l0], kShareCap);
      int cb = 0, ca = 0;  // valid entries of the two lists
      for (int i = lane; i < nb; i += 64) {
        lead[wave][i] = B[i];
        cb += B[i] >= 0;
      }
      wave_sync();
      for (int i = lane; i < na; i += 64) {
        const int x = A[i];
        if (x < 0) continue;
        ++ca;
        int lo = 0, hi = nb;
        while (lo < hi) {
          const int mid = (lo + hi) >> 1;
          const int v = lead[wave][mid];
          if (v >= 0 && v < x) lo = mid + 1;
          else hi = mid;
        }
        common += lo < nb && lead[wave][lo] == x;
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        ca += __shfl_xor(ca, o, 64);
        cb += __shfl_xor(cb, o, 64);
      }
      if (lane == 0) total = min(ca, cb);  // summed over the wave below
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    common += __shfl_xor(common, o, 64);
    total += __shfl_xor(total, o, 64);
  }
  if (lane == 0) {
    red[0][wave] = common;
    red[1][wave] = total;
  }
  __syncthreads();
  unsigned long long* acc = reinterpret_cast<unsigned long long*>(share + 2);
  unsigned int* ticket = reinterpret_cast<unsigned int*>(share + 6);
  if (threadIdx.x == 0) {
    atomicAdd(&acc[0], (unsigned long long)(red[0][0] + red[0][1] + red[0][2] + red[0][3]));
    atomicAdd(&acc[1], (unsigned long long)(red[1][0] + red[1][1] + red[1][2] + red[1][3]));
    __threadfence();  // the sums are visible before the ticket is taken
    last = atomicAdd(ticket, 1u) == gridDim.x - 1;
  }
  __syncthreads();
  if (last && threadIdx.x == 0) {
    __threadfence();
    const unsigned long long c = atomicAdd(&acc[0], 0ull);
    const unsigned long long n = atomicAdd(&acc[1], 0ull);
    share[0] = (n > 0 && 2 * c >= n) ? 1 : 0;
  }
}

hipError_t launch_prep_vertical(const AttnParams& p, int n_lists, const int* v_ptr, const int* v_idx,
                                hipStream_t st) {
  if (n_lists == 0) return hipSuccess;
  VS_TRACED(st, "vs_prep_vertical", hipLaunchKernelGGL(vs_prep_vertical_kernel, dim3(n_lists), dim3(kPrepThreads), 0, st, p, v_ptr, v_idx));
  if (p.map_group) {
    const int n_sample = std::min(n_lists, kShareSample);
    VS_TRACED(st, "vs_group_share", hipLaunchKernelGGL(vs_group_share_kernel, dim3((unsigned)((n_sample + 3) / 4)), dim3(256), 0, st, p, p.map_group));
  }
  return hipGetLastError();
}

// lse2 = LSE * log2(e): the backward recomputes P = exp(S - LSE) as
// exp2(S * scale * log2(e) - lse2).  An empty row (LSE = -inf) maps to +inf,
// so that P is 0 there whatever the scores.
__global__ __launch_bounds__(256) void vs_lse_log2_kernel(const float* lse, float* lse2, size_t count) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < count) {
    const float l = lse[i];
    lse2[i] = (l == -INFINITY) ? INFINITY : l * kLog2e;
  }
}

hipError_t launch_lse_log2(const float* lse, float* lse2, size_t count, hipStream_t st) {
  if (count == 0) return hipSuccess;
  VS_TRACED(st, "vs_lse_log2", hipLaunchKernelGGL(vs_lse_log2_kernel, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, st, lse, lse2, count));
  return hipGetLastError();
}

// delta[b, h, n] = sum_c dO[b, n, h, c] * O[b, n, h, c]  (MTraining §3.2 Eq. 1:
// rowsum(dA * A) = rowsum(dO * O)).  D/4 threads per row, 4 channels each;
// O and dO are addressed through their strides.
template <typename TO, typename TD, int D>
__global__ __launch_bounds__(256) void vs_delta_kernel(const TO* o, Stride3 so, const TD* dout, Stride3 sdo,
                                                       float* delta, int batch, int n, int h, size_t rows) {
  constexpr int TPR = D / 4;
  const size_t gt = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t row = gt / TPR;
  const int c4 = (int)(gt % TPR) * 4;
  // row = (b * n + pos) * h + head  ->  delta[(b * h + head) * n + pos]
  const size_t head = row % h;
  const size_t bp = row / h;
  const size_t pos = bp % n;
  const size_t b = bp / n;
  float acc = 0.f;
  if (row < rows) {
    const TO* orow = o + so.at(b, pos, head) + c4;
    const TD* drow = dout + sdo.at(b, pos, head) + c4;
#pragma unroll
    for (int u = 0; u < 4; ++u) acc += to_f32(orow[u]) * to_f32(drow[u]);
  }
#pragma unroll
  for (int w = TPR / 2; w >= 1; w >>= 1) acc += __shfl_xor(acc, w, 64);
  if (row < rows && (gt % TPR) == 0) delta[(b * h + head) * n + pos] = acc;
}

hipError_t launch_delta(const void* o, Stride3 so, int o_f32, int bf16, const void* dout, Stride3 sdo,
                        float* delta, int batch, int n, int h, int d, hipStream_t st) {
  const size_t rows = (size_t)batch * n * h;
  if (rows == 0) return hipSuccess;
  const size_t threads = rows * (d / 4);
  const dim3 grid((unsigned)((threads + 255) / 256));
#define VS_DELTA(TO, TD, DD)                                                                        \
  VS_TRACED(st, "vs_delta", hipLaunchKernelGGL((vs_delta_kernel<TO, TD, DD>), grid, dim3(256), 0, st, (const TO*)o, \
                     so, (const TD*)dout, sdo, delta, batch, n, h, rows))
  if (d == 128) {
    if (o_f32 && bf16) VS_DELTA(float, __bf16, 128);
    else if (o_f32) VS_DELTA(float, float, 128);
    else if (bf16) VS_DELTA(__bf16, __bf16, 128);
    else VS_DELTA(float, float, 128);
  } else {
    if (o_f32 && bf16) VS_DELTA(float, __bf16, 64);
    else if (o_f32) VS_DELTA(float, float, 64);
    else if (bf16) VS_DELTA(__bf16, __bf16, 64);
    else VS_DELTA(float, float, 64);
  }
#undef VS_DELTA
  return hipGetLastError();
}

// merge_out_and_lse (MTraining paper note, Algorithm 2), in place on the
// accumulator; a partial with LSE = -inf is the identity.  d/4 threads per
// row (one wave holds a whole row, so every lane reads lse_acc before any
// lane of the row writes it).
__global__ __launch_bounds__(256) void vs_lse_merge_kernel(int tpr, int n, int heads, size_t rows,
                                                           float* o_acc, float* lse_acc,
                                                           const float* o_part,
                                                           const float* lse_part) {
  const size_t gt = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t row = gt / tpr;
  if (row >= rows) return;
  const int c4 = (int)(gt % tpr) * 4;
  const size_t head = row % heads;
  const size_t bp = row / heads;
  const size_t pos = bp % n;
  const size_t b = bp / n;
  const size_t li = (b * heads + head) * n + pos;
  const float l1 = lse_acc[li];
  const float l2 = lse_part[li];
  const float mx = fmaxf(l1, l2);
  const size_t oi = row * (size_t)(tpr * 4) + c4;
  f32x4 r;
  float lse;
  if (mx == -INFINITY) {
    r = f32x4{0.f, 0.f, 0.f, 0.f};
    lse = -INFINITY;
  } else {
    const float w1 = expf(l1 - mx);
    const float w2 = expf(l2 - mx);
    const float tot = w1 + w2;
    lse = mx + logf(tot);
    const float a1 = w1 / tot;
    const float a2 = w2 / tot;
    const f32x4 x1 = *reinterpret_cast<const f32x4*>(o_acc + oi);
    const f32x4 x2 = *reinterpret_cast<const f32x4*>(o_part + oi);
    r = x1 * a1 + x2 * a2;
  }
  *reinterpret_cast<f32x4*>(o_acc + oi) = r;
  if (c4 == 0) lse_acc[li] = lse;
}

hipError_t launch_lse_merge(int batch, int n, int heads, int d, float* o_acc, float* lse_acc,
                            const float* o_part, const float* lse_part, hipStream_t st) {
  const size_t rows = (size_t)batch * n * heads;
  if (rows == 0) return hipSuccess;
  const int tpr = d / 4;
  const size_t threads = rows * tpr;
  VS_TRACED(st, "vs_lse_merge", hipLaunchKernelGGL(vs_lse_merge_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st,
                     tpr, n, heads, rows, o_acc, lse_acc, o_part, lse_part));
  return hipGetLastError();
}

}  // namespace vs
