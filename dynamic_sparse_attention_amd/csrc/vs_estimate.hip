// vs_estimate.hip — online Vertical-Slash index estimation.
//
// MTraining paper note, Algorithm 1 (first six steps) and MTraining §4.1
// (i)-(ii): the last query block of each segment is the observation window;
// its causal softmax A_hat over all keys of the segment gives the vertical
// scores (column sums, per token) and the slash scores (window mass on each
// block-diagonal of the 64x64 grid); argtopk keeps the highest of each, ties
// to the lowest index.
//
// gfx950 design, three passes over K plus a selection:
//   pass 1: one workgroup per (batch, KV head, 256-key tile); each wave takes
//           Q heads of the group, holds the 64 window rows as the B operand
//           and streams the tile's keys through S^T = K Q^T, keeping a
//           running (max, sum of exp) per row -> per-tile partials;
//   combine: per (list, row) the partials merge into the row's LSE;
//   pass 2: same grid, S = Q K^T so that a lane owns a key column; the
//           column sum of exp(S - LSE) is the vertical score and the sum
//           over a 64-key block is the slash score of its block-diagonal;
//   top-k:  one workgroup per (list, kind): 4-pass radix select on the fp32
//           score bits (scores are >= 0, so the bits order like the values),
//           with wave-aggregated histogram increments, then an ordered
//           compaction over contiguous per-wave ranges that writes the chosen
//           indices ascending, taking the lowest indices among scores equal
//           to the threshold.
#include <algorithm>

#include "vs_attn_common.h"
#include "vs_trace.h"

namespace vs {

constexpr int kEstKeyTile = 256;

struct TilePrefix {
  int v[129];
};

__device__ __forceinline__ int tile_seg(const TilePrefix& tp, int n_seg, int t) {
  int s = 0;
  while (s + 1 < n_seg && tp.v[s + 1] <= t) ++s;
  return s;
}

// This lane's part (channels hl * KPL + c * KC ..) of K row key_l.
template <typename T, int NCD, int KC, int KPL>
__device__ __forceinline__ void est_load_k(const T* kb, int kvs, int key_l, int hl,
                                           typename Mfma<T>::frag (&kf)[NCD]) {
  const T* kr = kb + (size_t)key_l * kvs;
#pragma unroll
  for (int c = 0; c < NCD; ++c) kf[c] = load_frag<T>(kr + c * KC + hl * KPL);
}

// bf16: the workgroup's kEstKeyTile K rows staged in LDS once by direct
// loads and read by every wave for each of its heads (instead of each wave
// fetching them from memory per head).  Row r's 16-byte chunk c sits at
// chunk index c ^ swz(r), so the 16 lanes of a fragment read (16 rows, one
// chunk) touch 16 distinct bank groups; rows past the tile's end repeat its
// last row (masked, as the memory path's clamped loads are).
template <int D>
struct EstKTile {
  static constexpr int CPR = D / 8;          // 16-byte chunks per row
  static constexpr int RPI = 64 / CPR;       // rows per 1 KiB direct load
  static constexpr int NI = kEstKeyTile / RPI;
  static constexpr int BYTES = kEstKeyTile * D * 2;
  __device__ static __forceinline__ int swz(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
  __device__ static __forceinline__ int off(int r, int c) { return r * CPR * 16 + 16 * (c ^ swz(r)); }

  // rows k0 .. k0 + kEstKeyTile - 1 of K (clamped to k1 - 1); every wave of
  // the workgroup issues NI / 4 loads, then waits and meets the others
  __device__ static __forceinline__ void stage(char* tile, const __bf16* kb, int kvs, int k0, int k1) {
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int rsub = lane / CPR;
#pragma unroll
    for (int u0 = 0; u0 < NI / 4; ++u0) {
      const int u = w * (NI / 4) + u0;
      const int r = u * RPI + rsub;
      const int key = min(k0 + r, k1 - 1);
      const int lc = (lane % CPR) ^ swz(r);
      dma_lds16(kb + (size_t)key * kvs + lc * 8, tile + u * 1024);
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_wait(0));
    __syncthreads();
  }

  // this lane's K operand of k chunk cc (channels 16 cc + 8 hl ..) for tile row r
  __device__ static __forceinline__ Mfma<__bf16>::frag frag(const char* tile, int r, int cc, int hl) {
    return *reinterpret_cast<const Mfma<__bf16>::frag*>(tile + off(r, 2 * cc + hl));
  }
};

template <typename T, int D>
__global__ __launch_bounds__(256) void vs_est_pass1_kernel(AttnParams p, TilePrefix tp, int tiles_total,
                                                           float2* part) {
  typedef Mfma<T> MF;
  typedef typename MF::frag frag;
  constexpr int KPL = MF::KPL, KC = 2 * KPL, NCD = D / KC;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, hl = lane >> 5, l32 = lane & 31;
  const int tg = blockIdx.x % tiles_total;
  const int bh = blockIdx.x / tiles_total;
  const int b = bh / p.h_kv, kvh = bh % p.h_kv;
  const int s = tile_seg(tp, p.seg.n_seg, tg);
  const int a = p.seg.start_blk[s] * kBlock, e = p.seg.start_blk[s + 1] * kBlock;
  const int k0 = a + (tg - tp.v[s]) * kEstKeyTile;
  const int k1 = min(k0 + kEstKeyTile, e);
  const int G = p.h_q / p.h_kv;
  const int kvs = (int)p.sk.t;
  const T* kb = reinterpret_cast<const T*>(p.k) + p.sk.at(b, 0, kvh);
  const T* q = reinterpret_cast<const T*>(p.q);
  constexpr bool kLds = sizeof(T) == 2;
  __shared__ __attribute__((aligned(16))) char ktile[kLds ? EstKTile<D>::BYTES : 16];
  if constexpr (kLds) EstKTile<D>::stage(ktile, reinterpret_cast<const __bf16*>(kb), kvs, k0, k1);
  for (int hg = wave; hg < G; hg += 4) {
    const int h = kvh * G + hg;
    frag qf[2][NCD];
#pragma unroll
    for (int rg = 0; rg < 2; ++rg) {
      const T* qr = q + p.sq.at(b, e - 64 + 32 * rg + l32, h);
#pragma unroll
      for (int c = 0; c < NCD; ++c) qf[rg][c] = load_frag<T>(qr + c * KC + hl * KPL);
    }
    float m[2] = {-INFINITY, -INFINITY}, l[2] = {0.f, 0.f};
    auto chunk = [&](int kc, const frag (&kf)[NCD]) {
#pragma unroll
      for (int rg = 0; rg < 2; ++rg) {
        f32x16 sc = f32x16{0};
#pragma unroll
        for (int c = 0; c < NCD; ++c) sc = MF::mma(kf[c], qf[rg][c], sc);
        const int row = e - 64 + 32 * rg + l32;
        float tt[16], mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kc + c_row(i, hl);
          tt[i] = (key < k1 && key <= row) ? sc[i] * p.sl2 : -INFINITY;
          mx = fmaxf(mx, tt[i]);
        }
        mx = half_max(mx);
        const float mn = fmaxf(m[rg], mx);
        const float mu = mn == -INFINITY ? 0.f : mn;
        float rs = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) rs += fast_exp2(tt[i] - mu);
        rs = half_sum(rs);
        l[rg] = l[rg] * fast_exp2(m[rg] - mu) + rs;
        m[rg] = mn;
      }
    };
    if constexpr (kLds) {
      // chunks of 32 keys from the staged tile
      for (int kc = k0; kc < k1; kc += 32) {
        frag kf[NCD];
#pragma unroll
        for (int c = 0; c < NCD; ++c) kf[c] = EstKTile<D>::frag(ktile, kc - k0 + l32, c, hl);
        chunk(kc, kf);
      }
    } else {
      // Chunks of 32 keys in pairs (a tile spans whole 64-key blocks), each
      // chunk's K rows loaded while the previous chunk computes.
      frag ka[NCD], kn[NCD];
      est_load_k<T, NCD, KC, KPL>(kb, kvs, min(k0 + l32, k1 - 1), hl, ka);
      for (int kc = k0; kc < k1; kc += 64) {
        est_load_k<T, NCD, KC, KPL>(kb, kvs, min(kc + 32 + l32, k1 - 1), hl, kn);
        chunk(kc, ka);
        if (kc + 64 < k1) est_load_k<T, NCD, KC, KPL>(kb, kvs, min(kc + 64 + l32, k1 - 1), hl, ka);
        chunk(kc + 32, kn);
      }
    }
    if (hl == 0) {
#pragma unroll
      for (int rg = 0; rg < 2; ++rg)
        part[(((size_t)b * p.h_q + h) * tiles_total + tg) * 64 + 32 * rg + l32] = make_float2(m[rg], l[rg]);
    }
  }
}

// Per (list, window row): merge the per-tile (max, sum of exp) partials into
// the row's LSE (log2 domain).  1024 threads per list: thread (group, row)
// merges the tiles t = group, group + 16, ... of its row, then the 16 group
// states of each row merge through LDS.
constexpr int kCombineGroups = 16;

__global__ __launch_bounds__(64 * kCombineGroups) void vs_est_combine_kernel(AttnParams p, TilePrefix tp, int tiles_total,
                                                            const float2* part, float* lse2) {
  __shared__ float2 st[kCombineGroups][64];
  const int list = blockIdx.x;
  const int s = list % p.seg.n_seg;
  const int bh = list / p.seg.n_seg;
  const int r = threadIdx.x & 63;
  const int grp = threadIdx.x >> 6;
  const float2* pp = part + (size_t)bh * tiles_total * 64;
  float M = -INFINITY, L = 0.f;
  for (int t = tp.v[s] + grp; t < tp.v[s + 1]; t += kCombineGroups) {
    const float2 v = pp[(size_t)t * 64 + r];
    const float mn = fmaxf(M, v.x);
    const float mu = mn == -INFINITY ? 0.f : mn;
    L = L * fast_exp2(M - mu) + v.y * fast_exp2(v.x - mu);
    M = mn;
  }
  st[grp][r] = make_float2(M, L);
  __syncthreads();
  if (grp == 0) {
    float Mg = -INFINITY;
#pragma unroll
    for (int g = 0; g < kCombineGroups; ++g) Mg = fmaxf(Mg, st[g][r].x);
    const float mu = Mg == -INFINITY ? 0.f : Mg;
    float Lg = 0.f;
#pragma unroll
    for (int g = 0; g < kCombineGroups; ++g) Lg += st[g][r].y * fast_exp2(st[g][r].x - mu);
    lse2[(size_t)list * 64 + r] = Lg > 0.f ? Mg + __log2f(Lg) : INFINITY;
  }
}

template <typename T, int D>
__global__ __launch_bounds__(256) void vs_est_pass2_kernel(AttnParams p, TilePrefix tp, int tiles_total,
                                                           const float* lse2, float* v_score,
                                                           float* s_score) {
  typedef Mfma<T> MF;
  typedef typename MF::frag frag;
  constexpr int KPL = MF::KPL, KC = 2 * KPL, NCD = D / KC;
  __shared__ float s_lse[4][64];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, hl = lane >> 5, l32 = lane & 31;
  const int tg = blockIdx.x % tiles_total;
  const int bh = blockIdx.x / tiles_total;
  const int b = bh / p.h_kv, kvh = bh % p.h_kv;
  const int s = tile_seg(tp, p.seg.n_seg, tg);
  const int a = p.seg.start_blk[s] * kBlock, e = p.seg.start_blk[s + 1] * kBlock;
  const int nb_s = (e - a) / kBlock;
  const int k0 = a + (tg - tp.v[s]) * kEstKeyTile;
  const int k1 = min(k0 + kEstKeyTile, e);
  const int G = p.h_q / p.h_kv;
  const int kvs = (int)p.sk.t;
  const int nbt = p.n_global / kBlock;
  const T* kb = reinterpret_cast<const T*>(p.k) + p.sk.at(b, 0, kvh);
  const T* q = reinterpret_cast<const T*>(p.q);
  constexpr bool kLds = sizeof(T) == 2;
  __shared__ __attribute__((aligned(16))) char ktile[kLds ? EstKTile<D>::BYTES : 16];
  if constexpr (kLds) EstKTile<D>::stage(ktile, reinterpret_cast<const __bf16*>(kb), kvs, k0, k1);
  for (int hg = wave; hg < G; hg += 4) {
    const int h = kvh * G + hg;
    const int list = (b * p.h_q + h) * p.seg.n_seg + s;
    s_lse[wave][lane] = lse2[(size_t)list * 64 + lane];
    wave_sync();
    // A operand: window rows in natural order (row slot m -> row e-64+32rg+m).
    frag qa[2][NCD];
#pragma unroll
    for (int rg = 0; rg < 2; ++rg) {
      const T* qr = q + p.sq.at(b, e - 64 + 32 * rg + l32, h);
#pragma unroll
      for (int c = 0; c < NCD; ++c) qa[rg][c] = load_frag<T>(qr + c * KC + hl * KPL);
    }
    float blk_acc = 0.f;
    // this lane's rows' LSE (log2 domain), held for the whole tile
    float lr[2][16];
#pragma unroll
    for (int rg = 0; rg < 2; ++rg)
#pragma unroll
      for (int i = 0; i < 16; ++i) lr[rg][i] = s_lse[wave][32 * rg + c_row(i, hl)];
    auto chunk = [&](int kc, const frag (&kf)[NCD]) {
      const int key = kc + l32;
      float col = 0.f;
#pragma unroll
      for (int rg = 0; rg < 2; ++rg) {
        f32x16 sc = f32x16{0};
#pragma unroll
        for (int c = 0; c < NCD; ++c) sc = MF::mma(qa[rg][c], kf[c], sc);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int rr = 32 * rg + c_row(i, hl);
          const int row = e - 64 + rr;
          col += (key < k1 && key <= row) ? fast_exp2(sc[i] * p.sl2 - lr[rg][i]) : 0.f;
        }
      }
      col = half_sum(col);
      if (hl == 0 && key < k1) v_score[((size_t)b * p.h_q + h) * p.n_global + key] = col;
      float bs = hl == 0 ? col : 0.f;
#pragma unroll
      for (int w = 16; w >= 1; w >>= 1) bs += __shfl_xor(bs, w, 64);
      blk_acc += bs;
      if (((kc - a) & 63) == 32) {  // second half of a 64-key block
        if (lane == 0) {
          const int beta = (kc - a) / kBlock;
          s_score[((size_t)b * p.h_q + h) * nbt + p.seg.start_blk[s] + (nb_s - 1 - beta)] = blk_acc;
        }
        blk_acc = 0.f;
      }
    };
    if constexpr (kLds) {
      for (int kc = k0; kc < k1; kc += 32) {
        frag kf[NCD];
#pragma unroll
        for (int c = 0; c < NCD; ++c) kf[c] = EstKTile<D>::frag(ktile, kc - k0 + l32, c, hl);
        chunk(kc, kf);
      }
    } else {
      // as in pass 1: chunk pairs, the next chunk's K rows loaded meanwhile
      frag ka[NCD], kn[NCD];
      est_load_k<T, NCD, KC, KPL>(kb, kvs, min(k0 + l32, k1 - 1), hl, ka);
      for (int kc = k0; kc < k1; kc += 64) {
        est_load_k<T, NCD, KC, KPL>(kb, kvs, min(kc + 32 + l32, k1 - 1), hl, kn);
        chunk(kc, ka);
        if (kc + 64 < k1) est_load_k<T, NCD, KC, KPL>(kb, kvs, min(kc + 64 + l32, k1 - 1), hl, ka);
        chunk(kc + 32, kn);
      }
    }
    wave_sync();
  }
}

constexpr int kTopkThreads = 1024;
constexpr int kTopkUnroll = 8;  // candidate loads per thread in flight

// Histogram increment of the active lanes' bins, aggregated per wave: the
// scores of a list cluster in a few bins of the leading digits, and lanes
// adding to one LDS word serialise.  Up to four distinct bins of the wave
// are added with one atomic each; the remaining lanes add their own.
__device__ __forceinline__ void wave_hist_add(int* hist, int bin, bool active) {
  const int lane = threadIdx.x & 63;
  uint64_t rem = __ballot(active);
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    if (rem == 0) break;  // uniform
    const int leader = __ffsll((unsigned long long)rem) - 1;
    const int lb = __shfl(bin, leader, 64);
    const uint64_t same = __ballot(active && bin == lb) & rem;
    if (lane == leader) atomicAdd(&hist[lb], __popcll(same));
    rem &= ~same;
  }
  if ((rem >> lane) & 1ull) atomicAdd(&hist[bin], 1);
}

// Run by the 64 lanes of one wave: the digit d of the kr-th largest active
// entry (counting from the top bin down, hist[d] the count of digit d, NB
// bins) and the rank kr - (entries in bins above d) inside that bin, into
// sel[0..1].  Lane l sums bins NB-1-PL*l .. NB-PL*(l+1) (PL = NB/64); a
// prefix over the lanes finds the lane whose bins reach kr, which then
// walks its PL.  (d = -1 if the bins hold fewer than kr entries.)
template <int NB = 256>
__device__ __forceinline__ void select_digit(const int* hist, int kr, int* sel) {
  constexpr int PL = NB / 64;
  const int lane = threadIdx.x & 63;
  int c[PL], own = 0;
#pragma unroll
  for (int q = 0; q < PL; ++q) {
    c[q] = hist[NB - 1 - PL * lane - q];
    own += c[q];
  }
  int incl = own;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
  const uint64_t hit = __ballot(incl >= kr);
  if (hit == 0) {
    if (lane == 63) {
      sel[0] = -1;
      sel[1] = kr - incl;
    }
    return;
  }
  if (lane == __ffsll((unsigned long long)hit) - 1) {
    int cum = incl - own, q = 0;
    for (; q < PL - 1; ++q) {
      if (cum + c[q] >= kr) break;
      cum += c[q];
    }
    sel[0] = NB - 1 - PL * lane - q;
    sel[1] = kr - cum;
  }
}

// Top-k selection (Algorithm 1, argtopk; ties to the lowest index): of the
// non-negative fp32 scores src[0..L) (whose bit patterns order as the
// values do) the k largest, emitted in index order as emit(pos, x, bits).
// The k-th largest value is found digit by digit (radix select); then the
// entries above it and the lowest-index entries equal to it are written:
// wave w owns the contiguous range [w C, (w + 1) C) of the list, counts
// its entries above / equal to it, and one workgroup scan gives every wave
// its output offset and its number of equal entries before it (ballot
// prefixes order the lanes of each 64-entry step).
constexpr int kTopkCand = 16384;   // LDS entries: a gathered bin, or merged candidates
constexpr int kTopkNW = kTopkThreads / 64;
constexpr int kTopkChunk = 16384;  // entries per first-stage workgroup of a long vertical list

struct TopkLds {
  int hist[256];
  int h1[2048];
  uint32_t cv[kTopkCand];
  int ci[kTopkCand];
  int wsum[2][kTopkNW];
  int wcnt[2][kTopkNW];
  int sel[2];
  int ncand;
};

// The write pass, once the k-th largest bit pattern `prefix`, the number kr
// of entries equal to it to take, and this wave's counts above / equal to it
// are known.
template <class Src, class Emit>
__device__ __forceinline__ void topk_write(TopkLds& S, Src src, int L, uint32_t prefix, int kr, int n_gt,
                                           int n_eq, Emit& emit) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int C = ((L + kTopkNW - 1) / kTopkNW + 63) & ~63;
  const int x0 = wave * C;
  const int x1 = min(x0 + C, L);
  const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  if (lane == 0) {
    S.wsum[0][wave] = n_gt;
    S.wsum[1][wave] = n_eq;
  }
  __syncthreads();
  int gt_before = 0, eq_before = 0;
  for (int w = 0; w < wave; ++w) {
    gt_before += S.wsum[0][w];
    eq_before += S.wsum[1][w];
  }
  int pos = gt_before + min(eq_before, kr);  // taken entries before this wave's range
  int eq_seen = eq_before;
  for (int xb0 = x0; xb0 < x1; xb0 += kTopkUnroll * 64) {  // wave-uniform trip count
    uint32_t vv[kTopkUnroll];
#pragma unroll
    for (int j = 0; j < kTopkUnroll; ++j) {
      const int x = xb0 + 64 * j + lane;
      vv[j] = x < x1 ? src(x) : 0u;
    }
#pragma unroll
    for (int j = 0; j < kTopkUnroll; ++j) {
      const int x = xb0 + 64 * j + lane;
      const uint32_t v = vv[j];
      const bool gt = x < x1 && v > prefix;
      const bool eq = x < x1 && v == prefix;
      const uint64_t meq = __ballot(eq);
      const bool take = gt || (eq && eq_seen + __popcll(meq & below) < kr);
      const uint64_t mt = __ballot(take);
      if (take) emit(pos + __popcll(mt & below), x, v);
      pos += __popcll(mt);
      eq_seen += __popcll(meq);
    }
  }
}

// Four 8-bit radix passes over the whole of src[0..L), then the counting and
// the write.
template <class Src, class Emit>
__device__ __forceinline__ void topk_radix4(TopkLds& S, Src src, int L, int k, Emit& emit) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  uint32_t prefix = 0, pmask = 0;
  int kr = k;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    if (tid < 256) S.hist[tid] = 0;
    __syncthreads();
    for (int base = 0; base < L; base += kTopkUnroll * kTopkThreads) {  // uniform trip count
      uint32_t v[kTopkUnroll];
#pragma unroll
      for (int j = 0; j < kTopkUnroll; ++j) {
        const int x = base + j * kTopkThreads + tid;
        v[j] = x < L ? src(x) : 0u;
      }
#pragma unroll
      for (int j = 0; j < kTopkUnroll; ++j) {
        const int x = base + j * kTopkThreads + tid;
        wave_hist_add(S.hist, (int)((v[j] >> shift) & 255), x < L && (v[j] & pmask) == prefix);
      }
    }
    __syncthreads();
    if (tid < 64) select_digit(S.hist, kr, S.sel);
    __syncthreads();
    prefix |= (uint32_t)S.sel[0] << shift;
    pmask |= 255u << shift;
    kr = S.sel[1];
    __syncthreads();
  }
  const int C = ((L + kTopkNW - 1) / kTopkNW + 63) & ~63;
  const int x0 = wave * C;
  const int x1 = min(x0 + C, L);
  int n_gt = 0, n_eq = 0;
  for (int xb = x0; xb < x1; xb += kTopkUnroll * 64) {
    uint32_t v[kTopkUnroll];
#pragma unroll
    for (int j = 0; j < kTopkUnroll; ++j) {
      const int x = xb + 64 * j + lane;
      v[j] = x < x1 ? src(x) : 0u;
    }
#pragma unroll
    for (int j = 0; j < kTopkUnroll; ++j) {
      const int x = xb + 64 * j + lane;
      n_gt += x < x1 && v[j] > prefix;
      n_eq += x < x1 && v[j] == prefix;
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    n_gt += __shfl_xor(n_gt, o, 64);
    n_eq += __shfl_xor(n_eq, o, 64);
  }
  topk_write(S, src, L, prefix, kr, n_gt, n_eq, emit);
}

// Scores in global memory: one pass over the leading 11 bits (2048 bins),
// one pass that counts per wave the entries above the k-th score's bin and
// gathers the bin's entries in LDS, the remaining 21 bits over the gathered
// entries only, and the write: three passes over the list.  A bin too full
// to gather takes topk_radix4 over the whole list.
template <class Emit>
__device__ __forceinline__ void topk_gather(TopkLds& S, const uint32_t* u, int L, int k, Emit& emit) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int C = ((L + kTopkNW - 1) / kTopkNW + 63) & ~63;
  const int x0 = wave * C;
  const int x1 = min(x0 + C, L);
  const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  auto gsrc = [u](int x) { return u[x]; };
  for (int x = tid; x < 2048; x += kTopkThreads) S.h1[x] = 0;
  if (tid < kTopkNW) {
    S.wcnt[0][tid] = 0;
    S.wcnt[1][tid] = 0;
  }
  if (tid == 0) S.ncand = 0;
  __syncthreads();
  for (int base = 0; base < L; base += kTopkUnroll * kTopkThreads) {
    uint32_t v[kTopkUnroll];
#pragma unroll
    for (int j = 0; j < kTopkUnroll; ++j) {
      const int x = base + j * kTopkThreads + tid;
      v[j] = x < L ? u[x] : 0u;
    }
#pragma unroll
    for (int j = 0; j < kTopkUnroll; ++j) wave_hist_add(S.h1, (int)(v[j] >> 21), base + j * kTopkThreads + tid < L);
  }
  __syncthreads();
  if (tid < 64) select_digit<2048>(S.h1, k, S.sel);
  __syncthreads();
  const uint32_t d1 = (uint32_t)S.sel[0];
  int kr = S.sel[1];
  int n_above = 0;
  for (int xb = x0; xb < x1; xb += kTopkUnroll * 64) {  // wave-uniform trip count
    uint32_t v[kTopkUnroll];
#pragma unroll
    for (int j = 0; j < kTopkUnroll; ++j) {
      const int x = xb + 64 * j + lane;
      v[j] = x < x1 ? u[x] : 0u;
    }
#pragma unroll
    for (int j = 0; j < kTopkUnroll; ++j) {
      const int x = xb + 64 * j + lane;
      const uint32_t dg = v[j] >> 21;
      n_above += x < x1 && dg > d1;
      const bool in = x < x1 && dg == d1;
      const uint64_t m = __ballot(in);
      if (m) {  // uniform
        int b0 = 0;
        if (lane == 0) b0 = atomicAdd(&S.ncand, __popcll(m));
        b0 = __shfl(b0, 0, 64);
        const int slot = b0 + __popcll(m & below);
        if (in && slot < kTopkCand) {
          S.cv[slot] = v[j];
          S.ci[slot] = x;
        }
      }
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) n_above += __shfl_xor(n_above, o, 64);
  __syncthreads();
  const int nc = S.ncand;
  if (nc > kTopkCand) {
    topk_radix4(S, gsrc, L, k, emit);
    return;
  }
  uint32_t prefix = d1 << 21, pmask = 0x7FFu << 21;
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 13 : (pass == 1 ? 5 : 0);
    const uint32_t wm = pass == 2 ? 31u : 255u;
    if (tid < 256) S.hist[tid] = 0;
    __syncthreads();
    for (int base = 0; base < nc; base += kTopkThreads) {  // uniform trip count
      const int i = base + tid;
      const uint32_t v = i < nc ? S.cv[i] : 0u;
      wave_hist_add(S.hist, (int)((v >> shift) & wm), i < nc && (v & pmask) == prefix);
    }
    __syncthreads();
    if (tid < 64) select_digit(S.hist, kr, S.sel);
    __syncthreads();
    prefix |= (uint32_t)S.sel[0] << shift;
    pmask |= wm << shift;
    kr = S.sel[1];
    __syncthreads();
  }
  for (int i = tid; i < nc; i += kTopkThreads) {
    const uint32_t v = S.cv[i];
    if (v > prefix) atomicAdd(&S.wcnt[0][S.ci[i] / C], 1);
    else if (v == prefix) atomicAdd(&S.wcnt[1][S.ci[i] / C], 1);
  }
  __syncthreads();
  topk_write(S, gsrc, L, prefix, kr, n_above + S.wcnt[0][wave], S.wcnt[1][wave], emit);
}

// The list (kind 0: vertical columns of a segment, kind 1: its
// block-diagonals) of workgroup pair 2 list + kind, its length, selection
// size and output.
struct TopkList {
  const uint32_t* u;
  int L, k, cap, add;
  int* out;
};
__device__ __forceinline__ TopkList topk_list(const AttnParams& p, const float* v_score, const float* s_score,
                                             const int* v_ptr, int* v_idx, const int* s_ptr, int* s_idx,
                                             const int* kcount, int list, int kind) {
  TopkList t;
  const int s = list % p.seg.n_seg;
  const int bh = list / p.seg.n_seg;
  const int a_blk = p.seg.start_blk[s];
  const int nb_s = p.seg.start_blk[s + 1] - a_blk;
  if (kind == 0) {
    t.u = reinterpret_cast<const uint32_t*>(v_score + (size_t)bh * p.n_global + (size_t)a_blk * kBlock);
    t.L = nb_s * kBlock;
    t.cap = v_ptr[list + 1] - v_ptr[list];
    t.out = v_idx ? v_idx + v_ptr[list] : nullptr;
    t.add = a_blk * kBlock;
  } else {
    t.u = reinterpret_cast<const uint32_t*>(s_score + (size_t)bh * (p.n_global / kBlock) + a_blk);
    t.L = nb_s;
    t.cap = s_ptr[list + 1] - s_ptr[list];
    t.out = s_idx + s_ptr[list];
    t.add = 0;
  }
  t.k = kcount ? min(kcount[2 * list + kind], t.cap) : t.cap;
  return t;
}

// A long vertical list is selected in two stages: each of nch >= 2 chunks
// of ch entries picks its own top-k (the global top-k, ties to the lowest
// index, lies in the union of the chunks' top-k: an entry that k others
// beat inside its chunk is beaten by them in the list), then the top-k of
// those candidates, which arrive in index order.  Chunks hold at most
// kTopkChunk entries, or fewer, longer ones where the nch * k candidates
// would not fit in LDS.
__device__ __forceinline__ bool topk_two_stage(const TopkList& t, int* nch, int* ch) {
  if (t.k <= 0 || t.k >= t.L) return false;
  int n = (t.L + kTopkChunk - 1) / kTopkChunk;
  if ((long long)n * t.k > kTopkCand) n = kTopkCand / t.k;
  *nch = n;
  *ch = (t.L + n - 1) / max(n, 1);
  return n >= 2;
}

// First stage: workgroup (list, chunk c) writes its chunk's top-min(k, len)
// entries (at most k <= kTopkCand / 2 < kTopkChunk), in index order, to
// cand[(list * nchunk + c) * kTopkChunk ...] as (score bits, index in the
// list) and their number to ccount; nchunk (the slots per list) is the
// longest list's kTopkChunk-entry chunk count, at least any list's nch.
__global__ __launch_bounds__(kTopkThreads) void vs_est_topk_chunk_kernel(AttnParams p, const float* v_score,
                                                                         const int* v_ptr, const int* kcount,
                                                                         int nchunk, uint2* cand, int* ccount) {
  __shared__ TopkLds S;
  const int list = blockIdx.x / nchunk;
  const int c = blockIdx.x % nchunk;
  const TopkList t = topk_list(p, v_score, nullptr, v_ptr, nullptr, nullptr, nullptr, kcount, list, 0);
  int nch, ch;
  if (!topk_two_stage(t, &nch, &ch) || c >= nch) return;
  const int x0 = c * ch;
  const int len = max(min(ch, t.L - x0), 0);
  uint2* dst = cand + ((size_t)list * nchunk + c) * kTopkChunk;
  if (threadIdx.x == 0) ccount[list * nchunk + c] = min(t.k, len);
  if (len == 0) return;
  auto emit = [dst, x0](int pos, int x, uint32_t v) { dst[pos] = make_uint2(v, (uint32_t)(x0 + x)); };
  if (t.k >= len) {
    for (int x = threadIdx.x; x < len; x += kTopkThreads) emit(x, x, t.u[x0 + x]);
    return;
  }
  topk_gather(S, t.u + x0, len, t.k, emit);
}

// kcount (optional): the number of entries to select per (list, kind), at
// most the list's capacity; the rest of the list is padded with -1.  Lists
// of the two-stage select merge their chunks' candidates (cand, ccount).
__global__ __launch_bounds__(kTopkThreads) void vs_est_topk_kernel(AttnParams p, const float* v_score,
                                                                   const float* s_score, const int* v_ptr,
                                                                   int* v_idx, const int* s_ptr,
                                                                   int* s_idx, const int* kcount, int nchunk,
                                                                   const uint2* cand, const int* ccount) {
  __shared__ TopkLds S;
  const int kind = blockIdx.x & 1;
  const int list = blockIdx.x >> 1;
  const TopkList t = topk_list(p, v_score, s_score, v_ptr, v_idx, s_ptr, s_idx, kcount, list, kind);
  const int tid = threadIdx.x;
  const int k = t.k, L = t.L, add = t.add;
  int* out = t.out;
  if (k >= L) {
    for (int x = tid; x < t.cap; x += kTopkThreads) out[x] = x < L ? x + add : -1;
    return;
  }
  if (k <= 0) {
    for (int x = tid; x < t.cap; x += kTopkThreads) out[x] = -1;
    return;
  }
  for (int x = k + tid; x < t.cap; x += kTopkThreads) out[x] = -1;
  int nch, ch;
  if (kind == 0 && cand && topk_two_stage(t, &nch, &ch)) {
    // the chunks' candidates, in index order, into LDS
    int nc = 0;
    for (int c = 0; c < nch; ++c) {
      const int m = ccount[list * nchunk + c];
      const uint2* src = cand + ((size_t)list * nchunk + c) * kTopkChunk;
      for (int i = tid; i < m; i += kTopkThreads) {
        const uint2 e = src[i];
        S.cv[nc + i] = e.x;
        S.ci[nc + i] = (int)e.y;
      }
      nc += m;
    }
    __syncthreads();
    const uint32_t* lcv = S.cv;
    auto lsrc = [lcv](int i) { return lcv[i]; };
    const int* lci = S.ci;
    auto emit = [out, add, lci](int pos, int i, uint32_t) { out[pos] = lci[i] + add; };
    topk_radix4(S, lsrc, nc, k, emit);
    return;
  }
  auto emit = [out, add](int pos, int x, uint32_t) { out[pos] = x + add; };
  topk_gather(S, t.u, L, k, emit);
}

// Top-p budgets (Algorithm 1, topp): per (list, kind) the fewest top scores,
// in (score desc, index asc) order, that hold a fraction p of the list's
// mass.  The decision is taken in integers, so it is exact and the same in
// every run: score s (fp32, >= 0) has mass m = rint(s * 2^54) (an observation
// window of at most 64 rows holds a mass of at most 64, so sums stay below
// 2^61); the target is T = ceil(t * total / 2^24) with t = rint(p * 2^24), p
// clamped to [0, 1]; k = the fewest entries whose masses reach T (0 when
// T = 0), capped by the list's capacity.  k is found by the four 8-bit radix
// passes of the top-k select with a mass histogram beside the count
// histogram (the crossing digit of each pass), over the entries at or above
// the cap-th largest score only, then the run of equal scores at the
// crossing.
__device__ __forceinline__ unsigned long long score_mass(uint32_t bits) {
  return (unsigned long long)__builtin_rint((double)__uint_as_float(bits) * 0x1p54);
}

// Count and mass histogram increments of the active lanes, aggregated per
// wave like wave_hist_add.
__device__ __forceinline__ void wave_mass_add(int* hc, unsigned long long* hm, int bin, bool active,
                                              unsigned long long m) {
  const int lane = threadIdx.x & 63;
  uint64_t rem = __ballot(active);
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    if (rem == 0) break;  // uniform
    const int leader = __ffsll((unsigned long long)rem) - 1;
    const int lb = __shfl(bin, leader, 64);
    const uint64_t same = __ballot(active && bin == lb) & rem;
    unsigned long long v = ((same >> lane) & 1ull) ? m : 0ull;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    if (lane == leader) {
      atomicAdd(&hc[lb], __popcll(same));
      atomicAdd(&hm[lb], v);
    }
    rem &= ~same;
  }
  if ((rem >> lane) & 1ull) {
    atomicAdd(&hc[bin], 1);
    atomicAdd(&hm[bin], m);
  }
}

__global__ __launch_bounds__(kTopkThreads) void vs_est_topp_kernel(AttnParams p, const float* v_score,
                                                                   const float* s_score, const int* v_ptr,
                                                                   const int* s_ptr, const float* p_v,
                                                                   const float* p_s, int* kcount) {
  __shared__ int hc[256];
  __shared__ unsigned long long hm[256];
  __shared__ unsigned long long red[kTopkThreads / 64];
  __shared__ unsigned long long red2[kTopkThreads / 64];
  __shared__ unsigned long long sel_need;
  __shared__ int sel_d, sel_above;
  __shared__ int sel2[2];
  const int kind = blockIdx.x & 1;
  const int list = blockIdx.x >> 1;
  const int s = list % p.seg.n_seg;
  const int bh = list / p.seg.n_seg;
  const int h = bh % p.h_q;
  const int a_blk = p.seg.start_blk[s];
  const int nb_s = p.seg.start_blk[s + 1] - a_blk;
  const int nbt = p.n_global / kBlock;
  const float* sc;
  int L, cap;
  float thr;
  if (kind == 0) {
    sc = v_score + (size_t)bh * p.n_global + (size_t)a_blk * kBlock;
    L = nb_s * kBlock;
    cap = v_ptr[list + 1] - v_ptr[list];
    thr = p_v[h];
  } else {
    sc = s_score + (size_t)bh * nbt + a_blk;
    L = nb_s;
    cap = s_ptr[list + 1] - s_ptr[list];
    thr = p_s[h];
  }
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const float pc = thr > 0.f ? fminf(thr, 1.f) : 0.f;  // NaN counts as 0
  const unsigned long long t = (unsigned long long)__builtin_rintf(pc * 16777216.f);
  if (cap <= 0 || t == 0 || L <= 0) {
    if (tid == 0) kcount[blockIdx.x] = 0;
    return;
  }
  const uint32_t* u = reinterpret_cast<const uint32_t*>(sc);
  // k never exceeds the capacity, so only entries at or above the cap-th
  // largest score kc can be selected: a count-only radix select (as in the
  // top-k select) finds kc, and the mass passes below look at those entries
  // only.
  uint32_t kc = 0;
  if (cap < L) {
    uint32_t pre = 0, pm = 0;
    int kr = cap;
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      if (tid < 256) hc[tid] = 0;
      __syncthreads();
      for (int base = 0; base < L; base += kTopkUnroll * kTopkThreads) {
        uint32_t v[kTopkUnroll];
#pragma unroll
        for (int j = 0; j < kTopkUnroll; ++j) {
          const int x = base + j * kTopkThreads + tid;
          v[j] = x < L ? u[x] : 0u;
        }
#pragma unroll
        for (int j = 0; j < kTopkUnroll; ++j) {
          const int x = base + j * kTopkThreads + tid;
          wave_hist_add(hc, (int)((v[j] >> shift) & 255), x < L && (v[j] & pm) == pre);
        }
      }
      __syncthreads();
      if (tid < 64) select_digit(hc, kr, sel2);
      __syncthreads();
      pre |= (uint32_t)sel2[0] << shift;
      pm |= 255u << shift;
      kr = sel2[1];
      __syncthreads();
    }
    kc = pre;
  }
  // total mass, and the mass of the entries >= kc (integer sums: exact in
  // any order)
  unsigned long long acc = 0, acc_ge = 0;
  for (int x = tid; x < L; x += kTopkThreads) {
    const uint32_t b = u[x];
    const unsigned long long m = score_mass(b);
    acc += m;
    acc_ge += b >= kc ? m : 0ull;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    acc += __shfl_xor(acc, o, 64);
    acc_ge += __shfl_xor(acc_ge, o, 64);
  }
  if (lane == 0) {
    red[wave] = acc;
    red2[wave] = acc_ge;
  }
  __syncthreads();
  unsigned long long total = 0, total_ge = 0;
#pragma unroll
  for (int w = 0; w < kTopkThreads / 64; ++w) {
    total += red[w];
    total_ge += red2[w];
  }
  if (total == 0) {
    if (tid == 0) kcount[blockIdx.x] = 0;
    return;
  }
  // T = ceil(t * total / 2^24) with total = hi 2^30 + lo (no product above 2^61)
  const unsigned long long hi = total >> 30, lo = total & ((1ull << 30) - 1);
  unsigned long long need = t * hi * 64ull + (t * lo + (1ull << 24) - 1) / (1ull << 24);
  if (need > total_ge) {
    // even every entry >= kc (at least cap of them) does not reach T
    if (tid == 0) kcount[blockIdx.x] = cap;
    return;
  }
  // Invariant: need <= the mass of the entries >= kc that match the prefix;
  // each pass picks the digit at which the mass of the larger entries
  // reaches it.
  uint32_t prefix = 0, pmask = 0;
  int above = 0, count_eq = 0;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    if (tid < 256) {
      hc[tid] = 0;
      hm[tid] = 0ull;
    }
    __syncthreads();
    for (int base = 0; base < L; base += kTopkUnroll * kTopkThreads) {
      uint32_t v[kTopkUnroll];
#pragma unroll
      for (int j = 0; j < kTopkUnroll; ++j) {
        const int x = base + j * kTopkThreads + tid;
        v[j] = x < L ? u[x] : 0u;
      }
#pragma unroll
      for (int j = 0; j < kTopkUnroll; ++j) {
        const int x = base + j * kTopkThreads + tid;
        const bool act = x < L && v[j] >= kc && (v[j] & pmask) == prefix;
        if (__ballot(act) == 0ull) continue;  // uniform
        wave_mass_add(hc, hm, (int)((v[j] >> shift) & 255), act, act ? score_mass(v[j]) : 0ull);
      }
    }
    __syncthreads();
    if (tid == 0) {
      unsigned long long cm = 0;
      int cc = 0, d = 255;
      for (; d > 0; --d) {
        if (cm + hm[d] >= need) break;
        cm += hm[d];
        cc += hc[d];
      }
      sel_d = d;
      sel_above = cc;
      sel_need = need - cm;
    }
    __syncthreads();
    prefix |= (uint32_t)sel_d << shift;
    pmask |= 255u << shift;
    above += sel_above;
    need = sel_need;
    count_eq = hc[sel_d];
    __syncthreads();
  }
  if (tid == 0) {
    // entries equal to the crossing score, in index order, each of mass ms
    const unsigned long long ms = score_mass(prefix);
    long long e = ms > 0 ? (long long)((need + ms - 1) / ms) : (long long)count_eq;
    e = e > count_eq ? count_eq : (e < 1 ? 1 : e);
    const long long k = (long long)above + e;
    kcount[blockIdx.x] = (int)(k < cap ? k : cap);
  }
}

hipError_t launch_estimate(const AttnParams& p, int dtype_bf16, int d, const int* v_ptr, int* v_idx,
                           const int* s_ptr, int* s_idx, float* v_score, float* s_score,
                           float2* partials, float* lse2, int tiles_total, const int* tile_prefix,
                           const float* p_v, const float* p_s, int* kcount, uint2* cand, int* ccount,
                           hipStream_t st) {
  TilePrefix tp;
  for (int s = 0; s <= p.seg.n_seg; ++s) tp.v[s] = tile_prefix[s];
  const int n_lists = p.batch * p.h_q * p.seg.n_seg;
  const dim3 g1((unsigned)(p.batch * p.h_kv * tiles_total));
#define VS_EST(T, DD)                                                                                   \
  do {                                                                                                  \
    VS_TRACED(st, "vs_est_pass1", hipLaunchKernelGGL((vs_est_pass1_kernel<T, DD>), g1, dim3(256), 0, st, p, tp, tiles_total, partials)); \
    VS_TRACED(st, "vs_est_combine", hipLaunchKernelGGL(vs_est_combine_kernel, dim3(n_lists), dim3(64 * kCombineGroups), 0, st, p, tp, tiles_total,        \
                       (const float2*)partials, lse2));                                                 \
    VS_TRACED(st, "vs_est_pass2", hipLaunchKernelGGL((vs_est_pass2_kernel<T, DD>), g1, dim3(256), 0, st, p, tp, tiles_total,          \
                       (const float*)lse2, v_score, s_score));                                           \
  } while (0)
  if (g1.x == 0) return hipSuccess;
  if (dtype_bf16 && d == 128) VS_EST(__bf16, 128);
  else if (dtype_bf16 && d == 64) VS_EST(__bf16, 64);
  else if (!dtype_bf16 && d == 128) VS_EST(float, 128);
  else VS_EST(float, 64);
#undef VS_EST
  if (p_v) {
    VS_TRACED(st, "vs_est_topp", hipLaunchKernelGGL(vs_est_topp_kernel, dim3(2 * n_lists), dim3(kTopkThreads), 0, st, p,
                       (const float*)v_score, (const float*)s_score, v_ptr, s_ptr, p_v, p_s, kcount));
  }
  // long vertical lists: a first stage per 16384-entry chunk
  int max_len = 0;
  for (int s = 0; s < p.seg.n_seg; ++s)
    max_len = std::max(max_len, (p.seg.start_blk[s + 1] - p.seg.start_blk[s]) * kBlock);
  const int nchunk = (max_len + kTopkChunk - 1) / kTopkChunk;
  const int* kc = p_v ? (const int*)kcount : (const int*)nullptr;
  if (nchunk >= 2 && cand)
    VS_TRACED(st, "vs_est_topk_chunk", hipLaunchKernelGGL(vs_est_topk_chunk_kernel, dim3(n_lists * nchunk), dim3(kTopkThreads), 0, st, p,
                       (const float*)v_score, v_ptr, kc, nchunk, cand, ccount));
  VS_TRACED(st, "vs_est_topk", hipLaunchKernelGGL(vs_est_topk_kernel, dim3(2 * n_lists), dim3(kTopkThreads), 0, st, p,
                     (const float*)v_score, (const float*)s_score, v_ptr, v_idx, s_ptr, s_idx, kc,
                     nchunk, (const uint2*)(nchunk >= 2 ? cand : nullptr), (const int*)ccount));
  return hipGetLastError();
}

}  // namespace vs
