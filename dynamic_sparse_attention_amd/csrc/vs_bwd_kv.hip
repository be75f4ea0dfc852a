// vs_bwd_kv.hip — dK / dV of the sparse backward, key-major, bf16 inputs.
//
// MTraining §3.2 Eq. 1-2 and the paper note's Appendix B.1: for the keys of a
// unit, dV += P^T dO and dK += scale * dS^T Q over every query row that reads
// them, with P = exp(S - LSE) recomputed from the final LSE and
// dS = P * (dP - delta), dP = dO V^T.
//
// A workgroup is two waves (four for pairs of key blocks and for column
// units); wave kh owns 32 keys (held as the B operands K^T,
// V^T) and accumulates dK^T, dV^T for them.  The query tiles the unit reads
// (64 rows of Q and dO of one Q head, plus their LSE * log2(e) and delta)
// stream through two LDS buffers: while the waves compute on one tile the
// next one arrives by direct global -> LDS loads (no registers, no packing).
// Q and dO are stored row-major with the 16-byte chunks of row r at chunk
// index c ^ f(r), f(r) = 2*(r % 4) + (r / 8) % 2.  The S = Q K^T and
// dP = dO V^T operands are 16-byte reads of rows {0-3, 8-11} + 4k by eight
// lanes at a time, the dK^T = Q^T dS and dV^T = dO^T P operands transposed
// reads (ds_read_b64_tr_b16) of four consecutive rows by sixteen lanes; f
// sends both to eight distinct 16-byte bank groups.
//
//   * slash units: (batch, KV head, key block j); the tiles are every
//     (Q head of the group, selected block-diagonal g) with query block j + g;
//     dK, dV of the block are complete at the end and are stored.  A grid too
//     small for the chip splits each key block's heads over 2 or 4 units,
//     which add their dK, dV with fp32 atomics into zeroed arrays.
//   * column units: (list, 128 gathered vertical columns, range of query
//     blocks); added to dK, dV with fp32 atomics after the slash kernel.
#include <algorithm>
#include <atomic>

#include "vs_attn_common.h"
#include "vs_trace.h"

namespace vs {

constexpr int kKvThreads = 128;
constexpr int kKvTiles = 512;  // tile list capacity per pass (query blocks)
constexpr int kTR = 32;        // query rows per staged tile: half a query block
// Waves (32 columns each) per column unit: four where whole lists are in
// the call, two for a striped call over one rank's key chunk, which holds
// about 1/W of each list's columns (there, units of 128 columns would leave
// half their waves without a column).
constexpr int kKvColWaves = 4, kKvColWavesChunk = 2;

template <int D>
struct RowTile {
  static constexpr int CPR = D / 8;          // 16-byte chunks per row
  static constexpr int RPI = 64 / CPR;       // rows per 1 KiB direct-load instruction
  static constexpr int BYTES = kTR * D * 2;  // kTR rows
  static constexpr int NDMA = kTR / RPI;     // direct-load instructions per tile
  __device__ static __forceinline__ constexpr int swz(int row) { return 2 * (row & 3) + ((row >> 3) & 1); }
  __device__ static __forceinline__ int off(int row, int chunk) {
    return (row / RPI) * 1024 + (row % RPI) * (CPR * 16) + 16 * (chunk ^ swz(row));
  }
};

template <int D>
struct __attribute__((aligned(16))) KvBuf {
  char q[RowTile<D>::BYTES];
  char dout[RowTile<D>::BYTES];
  float lse2[kTR];  // LSE * log2(e)
  float del[kTR];
  uint32_t sel[kTR];  // per-row block selection: the rows' picked blocks
};

typedef __attribute__((address_space(3))) void* lds_vptr;
typedef __attribute__((address_space(1))) void* glb_vptr;

// Direct loads of query tile (local block i, rows kTR*half .. +kTR, Q head h)
// into B; each of the NW waves issues its share of the rows (NDMA / NW
// instructions), waves 0 and 1 one of LSE / delta, and with SEL one wave
// (0, or 2 of four) also the rows' picked-block words of a per-row selection.
template <int D, bool SEL = false, int NW = 2>
__device__ __forceinline__ void kv_tile_dma(const AttnParams& p, KvBuf<D>& B, int b, int h, int i, int half) {
  typedef RowTile<D> RT;
  static_assert(RT::NDMA % NW == 0, "direct loads per tile must split evenly over the waves");
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int row0 = i * kBlock + kTR * half;  // first row of the tile in this batch row
  const __bf16* qb = reinterpret_cast<const __bf16*>(p.q) + p.sq.at(b, row0, h);
  const __bf16* db = reinterpret_cast<const __bf16*>(p.dout) + p.sdo.at(b, row0, h);
  const int rsub = lane / RT::CPR;
#pragma unroll
  for (int u0 = 0; u0 < RT::NDMA / NW; ++u0) {
    const int u = w * (RT::NDMA / NW) + u0;
    const int chunk = (lane % RT::CPR) ^ RT::swz(u * RT::RPI + rsub);
    const int rr = u * RT::RPI + rsub;  // row of the tile, < kTR
    __builtin_amdgcn_global_load_lds((glb_vptr)(qb + rr * p.sq.t + chunk * 8), (lds_vptr)(B.q + u * 1024), 16, 0, 0);
    __builtin_amdgcn_global_load_lds((glb_vptr)(db + rr * p.sdo.t + chunk * 8), (lds_vptr)(B.dout + u * 1024), 16, 0, 0);
  }
  const size_t li = ((size_t)b * p.h_q + h) * p.n_q + row0 + lane;
  const float* src = w == 0 ? p.lse2 : p.delta;
  if ((NW == 2 || w < 2) && lane < kTR)
    __builtin_amdgcn_global_load_lds((glb_vptr)(src + li), (lds_vptr)(w == 0 ? B.lse2 : B.del), 4, 0, 0);
  if (SEL && w == (NW == 2 ? 0 : 2) && lane < kTR)
    __builtin_amdgcn_global_load_lds((glb_vptr)(p.rmask + li), (lds_vptr)B.sel, 4, 0, 0);
}

template <int D>
struct KvWorkerB {
  typedef Mfma<__bf16> MF;
  typedef MF::frag frag;
  typedef RowTile<D> RT;
  static constexpr int KPL = 8, KC = 16;
  static constexpr int NCD = D / KC;   // k chunks over head_dim
  static constexpr int NCT = D / 32;   // 32-channel tiles of dK^T / dV^T
  static constexpr int DMA_PER_TILE = RT::NDMA + 1;  // per wave

  frag kB[NCD];     // B operand K^T of this lane's key column
  frag vB[NCD];     // B operand V^T
  f32x16 dk[NCT];   // dK^T [channel][key]
  f32x16 dv[NCT];   // dV^T [channel][key]

  __device__ __forceinline__ void load_keys(const AttnParams& p, int b, int kvh, int kpos) {
    const int hl = (threadIdx.x & 63) >> 5;
    const __bf16* kr = reinterpret_cast<const __bf16*>(p.k) + p.sk.at(b, kpos, kvh) + hl * KPL;
    const __bf16* vr = reinterpret_cast<const __bf16*>(p.v) + p.sv.at(b, kpos, kvh) + hl * KPL;
#pragma unroll
    for (int c = 0; c < NCD; ++c) {
      kB[c] = load_frag<__bf16>(kr + c * KC);
      vB[c] = load_frag<__bf16>(vr + c * KC);
    }
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      dk[ct] = f32x16{0};
      dv[ct] = f32x16{0};
    }
  }

  // LDS reads of a tile with per-lane offsets computed once, so that the
  // per-read part is a constant the ds_read offset field absorbs.  With the
  // row-major layout (row r at r * CPR * 16 bytes) and the chunk swizzle
  // c ^ swz(r), swz(r) < 8:
  //  * row operand (row 32rg + slot_perm(L%32), chunk 2c + L/32): the XOR
  //    only permutes chunks inside groups of 8, so the offset is
  //    ro[c % 4] + 32 * rg * CPR * 16 + 128 * (c / 4);
  //  * transposed operand (row 16c + 8h + 4q + (i/4) for lane i of a 16-lane
  //    group, chunk 4ct + x, x < 4): swz = 2(i/4) + h, so the chunk is
  //    4 (ct ^ zh) + zl with z = x ^ swz, and the offset is
  //    to[ct % 2] + 64 (ct - ct % 2) + (16c + 4q) * CPR * 16.
  int ro[4];
  int to[2];

  __device__ __forceinline__ void init_offsets() {
    const int lane = threadIdx.x & 63;
    const int hl = lane >> 5;
    const int sp = slot_perm<KPL>(lane & 31);
#pragma unroll
    for (int cl = 0; cl < 4; ++cl) ro[cl] = sp * (RT::CPR * 16) + 16 * ((2 * cl + hl) ^ RT::swz(sp));
    const int g = lane >> 4;
    const int sg = lane & 15;
    const int rr = sg >> 2;
    const int x = 2 * (g & 1) + ((sg & 3) >> 1);
    const int z = x ^ (2 * rr + hl);
    const int base = (8 * hl + rr) * (RT::CPR * 16) + 16 * (z & 3) + 8 * (sg & 1);
    to[0] = base + 64 * (z >> 2);
    to[1] = base + 64 * (1 - (z >> 2));
  }

  __device__ __forceinline__ frag row_frag(const char* t, int rg, int c) const {
    return *reinterpret_cast<const frag*>(t + ro[c & 3] + 32 * rg * (RT::CPR * 16) + 128 * (c >> 2));
  }

  // ds_read_b64_tr_b16: in each 16-lane group, lane i receives element i%4 of
  // the 8 bytes read by lanes i/4, 4+i/4, 8+i/4, 12+i/4 (rows k0 .. k0+3).
  __device__ __forceinline__ frag tr_frag(const char* t, int ct, int c) const {
    typedef short v4s __attribute__((ext_vector_type(4)));
    typedef short v8s __attribute__((ext_vector_type(8)));
    v4s part[2];
#pragma unroll
    for (int q = 0; q < 2; ++q)
      part[q] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(
          t + to[ct & 1] + 64 * (ct & ~1) + (16 * c + 4 * q) * (RT::CPR * 16)));
    const v8s both = __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(frag, both);
  }

  // One staged query tile of kTR = 32 rows (rows rbase .. rbase + 31 of the
  // query block).  kMasked: valid(r) says whether this lane's key column is
  // visible to row r of the block (else the tile is fully visible).  Masked
  // entries get exponent -inf, so P = dS = 0 there.
  template <bool kMasked, class ValidF>
  __device__ __forceinline__ void tile(const KvBuf<D>& B, float sl2, int rbase, ValidF valid) {
    const int lane = threadIdx.x & 63;
    const int hl = lane >> 5;
    f32x16 s = f32x16{0}, dp = f32x16{0};
#pragma unroll
    for (int c = 0; c < NCD; ++c) {
      s = MF::mma(row_frag(B.q, 0, c), kB[c], s);
      dp = MF::mma(row_frag(B.dout, 0, c), vB[c], dp);
    }
    frag pf[2], dsf[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      // register 8c + e holds tile row 16c + 8hl + e
      const int r0 = 16 * c + 8 * hl;
      const f32x4 la = *reinterpret_cast<const f32x4*>(B.lse2 + r0);
      const f32x4 lb = *reinterpret_cast<const f32x4*>(B.lse2 + r0 + 4);
      const f32x4 da = *reinterpret_cast<const f32x4*>(B.del + r0);
      const f32x4 db = *reinterpret_cast<const f32x4*>(B.del + r0 + 4);
      float pr[8], ds[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float l2 = e < 4 ? la[e] : lb[e - 4];
        const float dl = e < 4 ? da[e] : db[e - 4];
        float t = __builtin_fmaf(s[8 * c + e], sl2, -l2);
        if constexpr (kMasked) t = valid(rbase + r0 + e) ? t : -INFINITY;
        const float x = fast_exp2(t);
        pr[e] = x;
        ds[e] = x * (dp[8 * c + e] - dl);
      }
      pf[c] = MF::pack(pr);
      dsf[c] = MF::pack(ds);
    }
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        dv[ct] = MF::mma(tr_frag(B.dout, ct, c), pf[c], dv[ct]);
        dk[ct] = MF::mma(tr_frag(B.q, ct, c), dsf[c], dk[ct]);
      }
    }
  }

  // mode 0: store, 1: add (this thread owns the rows), 2: atomic add
  __device__ __forceinline__ void store(const AttnParams& p, int b, int kvh, int kpos, int mode) const {
    const int hl = (threadIdx.x & 63) >> 5;
    const size_t off = (((size_t)b * p.n_k + kpos) * p.h_kv + kvh) * D;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int ch = 32 * ct + 8 * i4 + 4 * hl;
        f32x4 a, v;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          a[u] = dk[ct][4 * i4 + u] * p.scale;
          v[u] = dv[ct][4 * i4 + u];
        }
        if (mode == 2) {
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            atomicAdd(p.dk + off + ch + u, a[u]);
            atomicAdd(p.dv + off + ch + u, v[u]);
          }
        } else if (mode == 1) {
          *reinterpret_cast<f32x4*>(p.dk + off + ch) += a;
          *reinterpret_cast<f32x4*>(p.dv + off + ch) += v;
        } else {
          *reinterpret_cast<f32x4*>(p.dk + off + ch) = a;
          *reinterpret_cast<f32x4*>(p.dv + off + ch) = v;
        }
      }
  }
};

template <int D, int NW = 2>
struct KvLdsB {
  KvBuf<D> buf[2];
  int tiles[kKvTiles];
  int wsum[NW];
};

// Double-buffered walk over ntiles query tiles: tile_of(t) -> (h, i, flags),
// body(B, t, flags) computes on the staged tile t.
// One pipeline step: the next tile's loads go to nxt while body computes on
// cur.  The two buffers never overlap; saying so (restrict) lets the compiler
// see that the reads of cur need not wait for the loads into nxt.
template <int D, bool SEL, int NW, class BodyF>
__device__ __forceinline__ void kv_step(const AttnParams& p, KvBuf<D>* __restrict__ nxt,
                                        const KvBuf<D>* __restrict__ cur, bool more, int b, int h1,
                                        int i1, int half1, int t, int fl, int half, BodyF& body) {
  if (more) kv_tile_dma<D, SEL, NW>(p, *nxt, b, h1, i1, half1);
  body(*cur, t, fl, half);
}

// Double-buffered walk over the two halves of ntiles query blocks:
// tile_of(t) -> (h, i, flags), body(B, t, flags, half) computes on the staged
// half tile.
template <int D, class TileF, class BodyF, bool SEL = false, int NW = 2>
__device__ __forceinline__ void kv_pipeline(const AttnParams& p, KvLdsB<D, NW>& L, int b, int ntiles,
                                            TileF tile_of, BodyF body) {
  if (ntiles == 0) return;
  int h, i, fl;
  tile_of(0, &h, &i, &fl);
  kv_tile_dma<D, SEL, NW>(p, L.buf[0], b, h, i, 0);
  const int nu = 2 * ntiles;
  for (int u = 0; u < nu; ++u) {
    // this wave's loads of step u are done; the barrier makes every wave's
    // loads visible and frees the other buffer (its step u-1 compute is over)
    __builtin_amdgcn_s_waitcnt(vmcnt_wait(0));
    __syncthreads();
    int h1 = 0, i1 = 0, fl1;
    const bool more = u + 1 < nu;
    if (more) tile_of((u + 1) >> 1, &h1, &i1, &fl1);
    tile_of(u >> 1, &h, &i, &fl);
    kv_step<D, SEL, NW>(p, &L.buf[(u + 1) & 1], &L.buf[u & 1], more, b, h1, i1, (u + 1) & 1, u >> 1, fl,
                        u & 1, body);
  }
  __syncthreads();
}

// The Vertical-Slash lists: one key block per workgroup.
template <int D>
__global__ __launch_bounds__(kKvThreads) __attribute__((amdgpu_waves_per_eu(2))) void vs_bwd_kv_slash_bf16_kernel(AttnParams p) {
  typedef KvWorkerB<D> W;
  __shared__ KvLdsB<D> L;
  const int tid = threadIdx.x;
  const int kh = tid >> 6;
  const int l32 = tid & 31;
  const int BH = p.batch * p.h_kv;
  const int bh = blockIdx.x % BH;
  // part of the key block's heads (kv_parts workgroups per key block, the
  // parts of a key block next to each other so that the longest walks start
  // first)
  const int part = (blockIdx.x / BH) % p.kv_parts;
  const int j = blockIdx.x / BH / p.kv_parts;
  const int b = bh / p.h_kv;
  const int kvh = bh % p.h_kv;
  const int G = p.h_q / p.h_kv;
  const int hpp = (p.hh_hi - p.hh_lo) / p.kv_parts;  // heads per part
  const int hh_lo = p.hh_lo + part * hpp;
  const int hh_hi = hh_lo + hpp;
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
  const int kpos = j * kBlock + 32 * kh + l32;
  const int kin = 32 * kh + l32;

  static_assert(sizeof(L.buf) >= 2 * 32 * 33 * 4, "epilogue staging must fit in the tile buffers");
  W wk;
  wk.init_offsets();
  wk.load_keys(p, b, kvh, kpos);
  int count = 0;
  auto tile_of = [&](int t, int* h, int* i, int* fl) {
    const int v = L.tiles[t];
    *h = kvh * G + (v >> 26);
    *i = (v >> 1) & ((1 << 25) - 1);
    *fl = v & 1;
  };
  // Diagonal tiles (g = 0: causal inside the block) first, in a walk of their
  // own, so that the main walk has no masking at all.
  {
    int i = -1;
    if (tid >= hh_lo && tid < hh_hi) {
      const int list = (b * p.h_q + kvh * G + tid) * p.seg.n_seg + seg;
      const int sp0 = p.s_ptr[list];
      if (p.s_ptr[list + 1] > sp0 && p.s_idx[sp0] == 0) i = local_query_block(p, kb_glob);
    }
    int tot;
    const int slot = block_compact<kKvThreads>(i >= 0, L.wsum, &tot);
    if (i >= 0) L.tiles[slot] = (tid << 26) | (i << 1) | 1;
    __syncthreads();
    auto diag_body = [&](const KvBuf<D>& B, int, int, int half) {
      wk.template tile<true>(B, p.sl2, kTR * half, [&](int r) { return kin <= r; });
    };
    kv_pipeline<D>(p, L, b, tot, tile_of, diag_body);
  }
  auto body = [&](const KvBuf<D>& B, int, int, int half) {
    wk.template tile<false>(B, p.sl2, kTR * half, [](int) { return true; });
  };
  for (int hh = hh_lo; hh < hh_hi; ++hh) {
    const int list = (b * p.h_q + kvh * G + hh) * p.seg.n_seg + seg;
    // candidates: the head's selected block-diagonals g > 0 (query block kb + g)
    const int sp0 = p.s_ptr[list];
    const int ns = p.s_ptr[list + 1] - sp0;
    for (int base = 0; base < ns; base += kKvThreads) {
      const int e = base + tid;
      int i = -1;
      if (e < ns) {
        const int g = p.s_idx[sp0 + e];
        if (g > 0 && beta_k + g < nb_seg) i = local_query_block(p, kb_glob + g);
      }
      int tot;
      const int slot = block_compact<kKvThreads>(i >= 0, L.wsum, &tot);
      if (i >= 0) L.tiles[count + slot] = (hh << 26) | (i << 1);
      count += tot;
      __syncthreads();
      if (count > kKvTiles - kKvThreads) {
        kv_pipeline<D>(p, L, b, count, tile_of, body);
        count = 0;
      }
    }
  }
  kv_pipeline<D>(p, L, b, count, tile_of, body);
  if (p.kv_parts == 1) {
    wk.store(p, b, kvh, kpos, p.kv_accumulate ? 1 : 0);
    return;
  }
  // Several parts add into the same keys: fp32 atomics into the zeroed (or
  // accumulating) dK, dV, staged through LDS (the tile buffers are free after
  // the walk's last barrier) one 32-channel slice at a time, so that every
  // atomic instruction covers 32 consecutive channels of two key rows.
  float* st = reinterpret_cast<float*>(reinterpret_cast<char*>(&L.buf[0]) + kh * 32 * 33 * 4);
  const size_t rstride = (size_t)p.h_kv * D;
  const size_t row0 = (((size_t)b * p.n_k + (size_t)j * kBlock + 32 * kh) * p.h_kv + kvh) * D;
  float* const gdst[2] = {p.dk + row0, p.dv + row0};
  const int hl = (tid & 63) >> 5;
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int ct = 0; ct < W::NCT; ++ct) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        st[l32 * 33 + c_row(i, hl)] = t == 0 ? wk.dk[ct][i] * p.scale : wk.dv[ct][i];
      wave_sync();
#pragma unroll 4
      for (int r = hl; r < 32; r += 2) atomicAdd(gdst[t] + (size_t)r * rstride + 32 * ct + l32, st[r * 33 + l32]);
      wave_sync();
    }
}

// MODE of the paired kernel below: a block selection (p.bmask) or a per-row
// block selection (p.rmask), both of one segment.
constexpr int kModeBlocks = 1, kModeRows = 2;

// Block and per-row selections (one segment): a workgroup of four waves owns
// the key blocks kb0 = 2 jp and kb0 + 1 (waves 2 kp + kh hold keys
// 32 kh .. +31 of block kb0 + kp).  Where both blocks lie in one selection
// block (always for 128-token block selections, and for per-row selections
// of 128 tokens or more, as the MoBA gate's), a later query block is
// selected for both or for neither and every staged Q / dO tile serves all
// four waves: half the tile loads of one block per workgroup.  (A per-row
// selection of 64-token blocks stages the query blocks either block picked,
// each wave masking the rows by its own block's bit.)  The diagonal
// walk stages query blocks kb0 and kb0 + 1 (causal inside their own key
// block, fully visible to kb0 from kb0 + 1, invisible to kb0 + 1 from kb0);
// the main walk the query blocks after kb0 + 1.  With an odd block count the
// second block of the last pair is absent: its waves take part in the loads
// and barriers only.
constexpr int kKvPairThreads = 256;

template <int D, int MODE>
__global__ __launch_bounds__(kKvPairThreads) __attribute__((amdgpu_waves_per_eu(2))) void vs_bwd_kv_pair_bf16_kernel(AttnParams p) {
  static_assert(MODE == kModeBlocks || MODE == kModeRows, "pairs serve block and per-row selections");
  constexpr bool ROWS = MODE == kModeRows;
  constexpr int NW = kKvPairThreads / 64;
  typedef KvWorkerB<D> W;
  __shared__ KvLdsB<D, NW> L;
  const int tid = threadIdx.x;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kh = wv & 1;
  const int kp = wv >> 1;
  const int l32 = tid & 31;
  const int BH = p.batch * p.h_kv;
  const int bh = blockIdx.x % BH;
  const int jp = blockIdx.x / BH;
  const int b = bh / p.h_kv;
  const int kvh = bh % p.h_kv;
  const int G = p.h_q / p.h_kv;
  const int nb = p.nkb;  // one segment: local = global blocks
  const int kb0 = 2 * jp;
  const int kbw = kb0 + kp;  // this wave's key block
  const bool live = kbw < nb;
  const int kin = 32 * kh + l32;
  const int kpos = (live ? kbw : kb0) * kBlock + kin;  // an absent block reads kb0's keys, unused
  // per-row selections: this wave's picked-block bit, and both blocks' bits
  const int pick = ROWS ? (kbw >> p.rm_shift) : 0;
  const uint32_t picks = ROWS ? ((1u << (kb0 >> p.rm_shift)) | (1u << ((kb0 + 1) >> p.rm_shift))) : 0u;

  W wk;
  wk.init_offsets();
  wk.load_keys(p, b, kvh, kpos);
  auto tile_of = [&](int t, int* h, int* i, int* fl) {
    const int v = L.tiles[t];
    *h = kvh * G + (v >> 26);
    *i = (v >> 1) & ((1 << 25) - 1);
    *fl = v & 1;
  };
  auto selected = [&](int list, int ib) -> bool {
    if (ROWS) return (p.rm_union[(size_t)list * p.nqb + ib] & picks) != 0u;
    return bmask_bit(p, list, ib >> 1, jp);
  };
  // diagonal walk: query blocks kb0 and kb0 + 1 of every head of the group
  {
    const int nd = p.hh_hi - p.hh_lo;
    int i = -1, hh = 0;
    if (tid < 2 * nd) {
      hh = p.hh_lo + (tid >> 1);
      const int ib = kb0 + (tid & 1);
      const int list = b * p.h_q + kvh * G + hh;
      if (ib < nb && selected(list, ib)) i = ib;
    }
    int tot;
    const int slot = block_compact<kKvPairThreads>(i >= 0, L.wsum, &tot);
    if (i >= 0) L.tiles[slot] = (hh << 26) | (i << 1) | 1;
    __syncthreads();
    auto diag_body = [&](const KvBuf<D>& B, int t, int, int half) {
      const int ib = (L.tiles[t] >> 1) & ((1 << 25) - 1);
      const int off = kin + kBlock * (kbw - ib);  // key position relative to the tile's rows
      if (!live || kbw > ib) return;              // no row of this tile sees the wave's keys
      if constexpr (ROWS)
        wk.template tile<true>(B, p.sl2, kTR * half, [&](int r) {
          return off <= r && ((B.sel[r - kTR * half] >> pick) & 1u) != 0u;
        });
      else
        wk.template tile<true>(B, p.sl2, kTR * half, [&](int r) { return off <= r; });
    };
    kv_pipeline<D, decltype(tile_of), decltype(diag_body), ROWS, NW>(p, L, b, tot, tile_of, diag_body);
  }
  // main walk: the selected query blocks after kb0 + 1, fully visible to both
  // blocks (with a per-row selection masked by the rows' picks)
  auto body = [&](const KvBuf<D>& B, int, int, int half) {
    if (!live) return;
    if constexpr (ROWS)
      wk.template tile<true>(B, p.sl2, kTR * half,
                             [&](int r) { return ((B.sel[r - kTR * half] >> pick) & 1u) != 0u; });
    else
      wk.template tile<false>(B, p.sl2, kTR * half, [](int) { return true; });
  };
  int count = 0;
  const int ns = nb - kb0 - 2;
  for (int hh = p.hh_lo; hh < p.hh_hi; ++hh) {
    const int list = b * p.h_q + kvh * G + hh;
    for (int base = 0; base < ns; base += kKvPairThreads) {
      const int e = base + tid;
      int i = -1;
      if (e < ns && selected(list, kb0 + 2 + e)) i = kb0 + 2 + e;
      int tot;
      const int slot = block_compact<kKvPairThreads>(i >= 0, L.wsum, &tot);
      if (i >= 0) L.tiles[count + slot] = (hh << 26) | (i << 1);
      count += tot;
      __syncthreads();
      if (count > kKvTiles - kKvPairThreads) {
        kv_pipeline<D, decltype(tile_of), decltype(body), ROWS, NW>(p, L, b, count, tile_of, body);
        count = 0;
      }
    }
  }
  kv_pipeline<D, decltype(tile_of), decltype(body), ROWS, NW>(p, L, b, count, tile_of, body);
  if (live) wk.store(p, b, kvh, kpos, p.kv_accumulate ? 1 : 0);
}

// Column units of NW waves, 32 * NW gathered columns: every staged query
// tile serves all of them (four waves: the Q / dO tile requests of two
// waves' units halved).
template <int NW>
__host__ __device__ constexpr int kv_col_units(int col_tiles) {
  return (64 * col_tiles + 32 * NW - 1) / (32 * NW);
}

template <int D, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2))) void vs_bwd_kv_cols_bf16_kernel(AttnParams p) {
  constexpr int NT = 64 * NW;  // threads
  constexpr int NC = 32 * NW;  // columns per unit
  typedef KvWorkerB<D> W;
  __shared__ KvLdsB<D, NW> L;
  static_assert(sizeof(L.buf) + sizeof(L.tiles) >= NW * 32 * 33 * 4, "epilogue staging must fit in the unit's LDS");
  extern __shared__ uint32_t bits[];  // (nb_seg + 31) / 32 words, sized at launch
  const int tid = threadIdx.x;
  const int kh = tid >> 6;
  const int l32 = tid & 31;
  const int ctiles = kv_col_units<NW>(p.col_tiles);
  int u = blockIdx.x;
  const int qr = u % p.qranges;
  u /= p.qranges;
  const int ctile = u % ctiles;
  const int list = u / ctiles;
  const int vc = p.vcnt[list];
  if (NC * ctile >= vc) return;
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
  const int* vs = p.vsel + (size_t)list * p.vsel_stride + NC * ctile;
  const int ncol = min(NC, vc - NC * ctile);
  const int first_blk = vs[0] / kBlock;  // global block of the first column
  // first local query block whose global block is >= first_blk
  int i_first = p.W == 1 ? first_blk : (first_blk <= p.q_rank ? 0 : (first_blk - p.q_rank + p.W - 1) / p.W);
  const int r_lo = max(max(i_lo, qr * p.qrange_len), i_first);
  const int r_hi = min(i_hi, (qr + 1) * p.qrange_len);
  if (r_lo >= r_hi) return;

  // This lane's column, or (past the unit's columns) a position after every
  // row, which no row sees; the walk keeps only this one value per lane.
  const int col = 32 * kh + l32;
  const bool col_ok = col < ncol;
  const int m = col_ok ? vs[col] : 0x3fffffff;

  const int sp0 = p.s_ptr[list];
  const int ns = p.s_ptr[list + 1] - sp0;
  const int nwords = (nb_seg + 31) >> 5;
  for (int w = tid; w < nwords; w += NT) bits[w] = 0u;
  __syncthreads();
  for (int e = tid; e < ns; e += NT) {
    const int g = p.s_idx[sp0 + e];
    if (g >= 0 && g < nb_seg) atomicOr(&bits[g >> 5], 1u << (g & 31));
  }
  __syncthreads();

  W wk;
  wk.init_offsets();
  wk.load_keys(p, b, kvh, local_key_pos(p, vs[col_ok ? col : 0]));
  auto qglob = [&](int i) { return p.W == 1 ? i : p.q_rank + p.W * i; };
  auto tile_of = [&](int t, int* hh, int* i, int* fl) {
    *hh = h;
    *i = r_lo + t;
    *fl = 0;
  };
  const int ntiles = r_hi - r_lo;
  auto body = [&](const KvBuf<D>& B, int t, int, int half) {
    const int qbg = qglob(r_lo + t);
    const int beta_q = qbg - a_blk;
    const int off = beta_q - ((m >> 6) - a_blk);  // block-diagonal of (query block, column)
    const bool lane_ok = off >= 0 && ((bits[off >> 5] >> (off & 31)) & 1u) == 0u;
    const int row0 = qbg * kBlock;
    const int mr = lane_ok ? m - row0 : 64;  // first visible row
    wk.template tile<true>(B, p.sl2, kTR * half, [&](int r) { return mr <= r; });
  };
  kv_pipeline<D, decltype(tile_of), decltype(body), false, NW>(p, L, b, ntiles, tile_of, body);
  // Add this wave's dK, dV columns into the gradients, staged through LDS
  // (the tile buffers are free now) one 32-channel slice at a time, so that
  // each atomic instruction covers 32 consecutive channels of two key rows
  // rather than single channels of 32 different rows.
  const int kpos = local_key_pos(p, vs[col_ok ? col : 0]);
  float* st = reinterpret_cast<float*>(reinterpret_cast<char*>(&L.buf[0]) + kh * 32 * 33 * 4);
  const int nvalid = min(max(ncol - 32 * kh, 0), 32);
  const size_t rstride = (size_t)p.h_kv * D;
  float* const gdst[2] = {p.dk + ((size_t)b * p.n_k * p.h_kv + kvh) * D,
                          p.dv + ((size_t)b * p.n_k * p.h_kv + kvh) * D};
  const int hl = (tid & 63) >> 5;
  const int c32 = tid & 31;
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int ct = 0; ct < W::NCT; ++ct) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        st[l32 * 33 + c_row(i, hl)] = t == 0 ? wk.dk[ct][i] * p.scale : wk.dv[ct][i];
      wave_sync();
      for (int r = hl; r < nvalid; r += 2) {
        const int kr = __shfl(kpos, r, 64);
        atomicAdd(gdst[t] + (size_t)kr * rstride + 32 * ct + c32, st[r * 33 + c32]);
      }
      wave_sync();
    }
}

// dK = dV = 0 before slash units that add with atomics (a kernel rather than
// a memset, so that the call can be captured in a graph).
__global__ __launch_bounds__(256) void vs_zero2_kernel(f32x4* a, f32x4* c, size_t n4) {
  for (size_t x = (size_t)blockIdx.x * 256 + threadIdx.x; x < n4; x += (size_t)gridDim.x * 256) {
    a[x] = f32x4{0.f, 0.f, 0.f, 0.f};
    c[x] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
}

// Compute units of the current device (cached per device; calls from
// several host threads may both look it up and store the same value).
static int device_cus() {
  static std::atomic<int> cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Workgroups per key block of the slash dK/dV kernel.  A unit's walk is
// proportional to the block-diagonals that still fit after its key block, so
// the earliest key blocks walk the longest; a grid of fewer than two rounds
// of resident workgroups (four per CU) finishes with the longest walk, on a
// chip mostly idle.  There the heads of a key block are split over parts (a
// power of two dividing the group, at most 4), whose results add with
// atomics.
static int slash_parts(const AttnParams& p, unsigned units) {
  const int G = (p.hh_hi - p.hh_lo);
  const long rounds2 = 2L * 4 * device_cus();
  int parts = 1;
  while (parts < 4 && (long)units * parts < rounds2 && G % (2 * parts) == 0) parts *= 2;
  return parts;
}

hipError_t launch_bwd_kv_bf16(const AttnParams& p0, int d, hipStream_t st) {
  AttnParams p = p0;
  const dim3 gs((unsigned)(p.batch * p.h_kv * p.nkb));
  const bool chunk = p.W > 1 && !p.k_all;
  const int ucols = p.batch * p.h_q * p.seg.n_seg * p.qranges;
  const dim3 gc((unsigned)(ucols * (chunk ? kv_col_units<kKvColWavesChunk>(p.col_tiles)
                                           : kv_col_units<kKvColWaves>(p.col_tiles))));
  p.hh_lo = 0;
  p.hh_hi = p.h_q / p.h_kv;
  p.kv_accumulate = 0;
  p.kv_parts = (p.bmask || p.rmask) ? 1 : slash_parts(p, gs.x);
  const dim3 gsp(gs.x * p.kv_parts);
  if (gs.x && p.kv_parts > 1) {
    const size_t n4 = (size_t)p.batch * p.n_k * p.h_kv * d / 4;
    const unsigned zb = (unsigned)std::min<size_t>((n4 + 255) / 256, 8192);
    VS_TRACED(st, "vs_zero_dkdv", hipLaunchKernelGGL(vs_zero2_kernel, dim3(zb), dim3(256), 0, st,
                                                      reinterpret_cast<f32x4*>(p.dk), reinterpret_cast<f32x4*>(p.dv), n4));
  }
  // bitmap of the selected block-diagonals: one bit per block of the longest segment
  int nb_max = p.W == 1 ? 0 : p.n_global / kBlock;
  for (int sgi = 0; p.W == 1 && sgi < p.seg.n_seg; ++sgi)
    nb_max = std::max(nb_max, p.seg.start_blk[sgi + 1] - p.seg.start_blk[sgi]);
  const size_t bits_bytes = (size_t)((nb_max + 31) / 32) * 4 + 4;
  // block and per-row selections: pairs of key blocks per workgroup
  const dim3 gp((unsigned)(p.batch * p.h_kv * ((p.nkb + 1) / 2)));
  if (d == 128) {
    if (gs.x && p.bmask) VS_TRACED(st, "vs_bwd_dkdv_slash", hipLaunchKernelGGL((vs_bwd_kv_pair_bf16_kernel<128, kModeBlocks>), gp, dim3(kKvPairThreads), 0, st, p));
    else if (gs.x && p.rmask) VS_TRACED(st, "vs_bwd_dkdv_slash", hipLaunchKernelGGL((vs_bwd_kv_pair_bf16_kernel<128, kModeRows>), gp, dim3(kKvPairThreads), 0, st, p));
    else if (gs.x) VS_TRACED(st, "vs_bwd_dkdv_slash", hipLaunchKernelGGL((vs_bwd_kv_slash_bf16_kernel<128>), gsp, dim3(kKvThreads), 0, st, p));
    if (gc.x && chunk) VS_TRACED(st, "vs_bwd_dkdv_cols", hipLaunchKernelGGL((vs_bwd_kv_cols_bf16_kernel<128, kKvColWavesChunk>), gc, dim3(64 * kKvColWavesChunk), bits_bytes, st, p));
    else if (gc.x) VS_TRACED(st, "vs_bwd_dkdv_cols", hipLaunchKernelGGL((vs_bwd_kv_cols_bf16_kernel<128, kKvColWaves>), gc, dim3(64 * kKvColWaves), bits_bytes, st, p));
  } else {
    if (gs.x && p.bmask) VS_TRACED(st, "vs_bwd_dkdv_slash", hipLaunchKernelGGL((vs_bwd_kv_pair_bf16_kernel<64, kModeBlocks>), gp, dim3(kKvPairThreads), 0, st, p));
    else if (gs.x && p.rmask) VS_TRACED(st, "vs_bwd_dkdv_slash", hipLaunchKernelGGL((vs_bwd_kv_pair_bf16_kernel<64, kModeRows>), gp, dim3(kKvPairThreads), 0, st, p));
    else if (gs.x) VS_TRACED(st, "vs_bwd_dkdv_slash", hipLaunchKernelGGL((vs_bwd_kv_slash_bf16_kernel<64>), gsp, dim3(kKvThreads), 0, st, p));
    if (gc.x && chunk) VS_TRACED(st, "vs_bwd_dkdv_cols", hipLaunchKernelGGL((vs_bwd_kv_cols_bf16_kernel<64, kKvColWavesChunk>), gc, dim3(64 * kKvColWavesChunk), bits_bytes, st, p));
    else if (gc.x) VS_TRACED(st, "vs_bwd_dkdv_cols", hipLaunchKernelGGL((vs_bwd_kv_cols_bf16_kernel<64, kKvColWaves>), gc, dim3(64 * kKvColWaves), bits_bytes, st, p));
  }
  return hipGetLastError();
}

}  // namespace vs
