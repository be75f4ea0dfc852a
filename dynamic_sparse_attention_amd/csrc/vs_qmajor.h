// vs_qmajor.h — query-major walk over the Vertical-Slash support of one
// query block, shared by the forward kernel and the dQ backward kernel.
//
// A workgroup owns one (batch, Q head, query block) and expands the index of
// the block on the fly (MTraining paper note, Algorithm 1 sparseformat and
// Algorithm 2 convert_index): first the selected block-diagonals become
// key-block tiles, then the selected vertical columns that are not inside a
// selected block become 64-column tiles.  The tiles are dealt round-robin to
// NS key streams.  The bf16 kernels run one stream of two waves (rows 0-31
// and 32-63, sharing every tile); the fp32 kernels run four streams of one
// wave each, every wave keeping a running state for all 64 rows, combined at
// the end.
#pragma once

#include "vs_attn_common.h"

namespace vs {

constexpr int kQThreads = 256;

// The half-tiles (32 keys) one key stream consumes from the current tile
// list: tiles wave, wave + NS, ... (round-robin over NS streams), two halves
// each.  key_pos(n, r): local key position of key r (0..31) of half-tile n;
// full(n): no masking needed; valid(n, e, r): key e of the half for row r.
template <int NS>
struct SlashSetT {
  static constexpr bool kContiguous = true;  // the 32 keys of a half are consecutive
  const int* tiles;  // 2 * local key block + (g == 0)
  int tot;
  int wave;          // key stream
  __device__ __forceinline__ int n_halves() const { return tot > wave ? 2 * ((tot - wave + NS - 1) / NS) : 0; }
  __device__ __forceinline__ int n_halves_max() const { return tot > 0 ? 2 * ((tot + NS - 1) / NS) : 0; }
  __device__ __forceinline__ int tv(int n) const { return tiles[wave + NS * (n >> 1)]; }
  __device__ __forceinline__ int key_pos(int n, int r) const { return (tv(n) >> 1) * kBlock + 32 * (n & 1) + r; }
  __device__ __forceinline__ bool full(int n) const { return (tv(n) & 1) == 0; }
  __device__ __forceinline__ bool valid(int n, int e, int r) const { return 32 * (n & 1) + e <= r; }
  // -inf where key reg_row(i, hl) of half n is not visible from row r
  template <int KPL>
  __device__ __forceinline__ void mask(int n, int hl, int r, f32x16& s) const {
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (!valid(n, reg_row<KPL>(i, hl), r)) s[i] = -INFINITY;
  }
};

// Key-block tiles of a per-row block selection: the rows of the query block
// that did not pick a tile's block see none of it.
template <int NS>
struct MobaSetT {
  static constexpr bool kContiguous = true;
  const int* tiles;      // 4 * local key block + 2 * (some row did not pick its block) + (diagonal)
  int tot;
  int wave;              // key stream
  const uint32_t* rsel;  // the 64 rows' picked blocks (one word per row)
  int shift;             // log2 of the 64-key blocks per picked block
  __device__ __forceinline__ int n_halves() const { return tot > wave ? 2 * ((tot - wave + NS - 1) / NS) : 0; }
  __device__ __forceinline__ int n_halves_max() const { return tot > 0 ? 2 * ((tot + NS - 1) / NS) : 0; }
  __device__ __forceinline__ int tv(int n) const { return tiles[wave + NS * (n >> 1)]; }
  __device__ __forceinline__ int key_pos(int n, int r) const { return (tv(n) >> 2) * kBlock + 32 * (n & 1) + r; }
  __device__ __forceinline__ bool full(int n) const { return (tv(n) & 3) == 0; }
  __device__ __forceinline__ bool picked(int n, int r) const { return (rsel[r] >> ((tv(n) >> 2) >> shift)) & 1u; }
  __device__ __forceinline__ bool valid(int n, int e, int r) const {
    return picked(n, r) && (!(tv(n) & 1) || 32 * (n & 1) + e <= r);
  }
  template <int KPL>
  __device__ __forceinline__ void mask(int n, int hl, int r, f32x16& s) const {
    const bool row_ok = picked(n, r);
    const bool diag = tv(n) & 1;
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (!row_ok || (diag && 32 * (n & 1) + reg_row<KPL>(i, hl) > r)) s[i] = -INFINITY;
  }
};

// Key-block tiles of a pair of query blocks 2I and 2I + 1 of one 128-row
// block (block selections, whose selection the two share): the
// pair's rows r = 0..127; key block 2I + d (d = 0, 1) is causal for row r
// (key offset 64 d + e visible iff <= r), earlier blocks are fully visible.
template <int NS>
struct PairSetT {
  static constexpr bool kContiguous = true;
  const int* tiles;  // 4 * local key block + 2 * (block 2I + 1) + (block 2I or 2I + 1)
  int tot;
  int wave;          // key stream
  __device__ __forceinline__ int n_halves() const { return tot > wave ? 2 * ((tot - wave + NS - 1) / NS) : 0; }
  __device__ __forceinline__ int n_halves_max() const { return tot > 0 ? 2 * ((tot + NS - 1) / NS) : 0; }
  __device__ __forceinline__ int tv(int n) const { return tiles[wave + NS * (n >> 1)]; }
  __device__ __forceinline__ int key_pos(int n, int r) const { return (tv(n) >> 2) * kBlock + 32 * (n & 1) + r; }
  __device__ __forceinline__ bool full(int n) const { return (tv(n) & 1) == 0; }
  __device__ __forceinline__ int koff(int n) const { return 64 * ((tv(n) >> 1) & 1) + 32 * (n & 1); }
  __device__ __forceinline__ bool valid(int n, int e, int r) const { return koff(n) + e <= r; }
  template <int KPL>
  __device__ __forceinline__ void mask(int n, int hl, int r, f32x16& s) const {
    const int k0 = koff(n);
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (k0 + reg_row<KPL>(i, hl) > r) s[i] = -INFINITY;
  }
};

template <int NS>
struct ColSetT {
  static constexpr bool kContiguous = false;
  const int* cols;   // local key positions of the gathered columns
  const int* coff;   // -1, or the first row (0..63) that may see the column (kBlock: none)
  int count;         // columns in the list
  int nt;            // 64-column tiles in the list
  int wave;          // key stream
  __device__ __forceinline__ int n_halves() const { return nt > wave ? 2 * ((nt - wave + NS - 1) / NS) : 0; }
  __device__ __forceinline__ int n_halves_max() const { return nt > 0 ? 2 * ((nt + NS - 1) / NS) : 0; }
  __device__ __forceinline__ int base(int n) const { return 64 * (wave + NS * (n >> 1)) + 32 * (n & 1); }
  // Entries past count up to the end of the last tile repeat a listed
  // column (qmajor_drive fills them), so every read is of a valid position.
  __device__ __forceinline__ int key_pos(int n, int r) const { return cols[base(n) + r]; }
  // Columns are in ascending position, so those with a per-row limit (inside
  // the query block) come last, then the padding (limit kBlock, seen by no
  // row): a half is unmasked if its last column has no limit.
  __device__ __forceinline__ bool full(int n) const { return coff[base(n) + 31] < 0; }
  __device__ __forceinline__ bool valid(int n, int e, int r) const { return coff[base(n) + e] <= r; }
  // -inf where key reg_row(i, hl) of half n is not visible from row r; the
  // limits of a lane's 16 keys are two runs of KPL = 8, read as four 16-byte
  // loads.
  template <int KPL>
  __device__ __forceinline__ void mask(int n, int hl, int r, f32x16& s) const {
    static_assert(KPL == 8, "bf16 operand layout");
    typedef int i32x4 __attribute__((ext_vector_type(4)));
    const i32x4* c = reinterpret_cast<const i32x4*>(coff + base(n) + hl * KPL);
    const i32x4 q[4] = {c[0], c[1], c[4], c[5]};
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (q[i / 4][i % 4] > r) s[i] = -INFINITY;
  }
};

// Selected vertical columns are gathered in batches of up to kColBatch
// (16 tiles of 64 columns, four per wave with 256 threads), so that each
// pipelined walk over a batch has several tiles per wave to overlap.
constexpr int kColBatch = 1024;

typedef SlashSetT<4> SlashSet;
typedef ColSetT<4> ColSet;

template <int NT = kQThreads, int NCOL = kColBatch>
struct QMajorLds {
  static constexpr int kCols = NCOL;
  int tiles[NT];
  alignas(16) int cols[NCOL];
  alignas(16) int coff[NCOL];
  int wsum[NT / 64];
};

// Block selections over a pair of query blocks rb.beta (even) and
// rb.beta + 1 (absent past the segment's end): the key blocks up to the
// pair's last block that its 128-row block selected.
template <int NS, int NT, int NCOL, class Worker>
__device__ __forceinline__ void qmajor_drive_pair(const AttnParams& p, const RowBlock& rb, int list,
                                                  QMajorLds<NT, NCOL>& L, Worker& wk) {
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane((tid >> 6) % NS);
  const int last = min(rb.beta + 1, rb.nb_seg - 1);  // the pair's last query block
  {
    const int bh = list;  // one segment: list = b * h_q + h
    for (int base = 0; base <= last; base += NT) {
      const int kb = base + tid;
      int j = -1;
      if (kb <= last && bmask_bit(p, bh, rb.beta >> 1, kb >> 1)) j = local_key_block(p, rb.a_blk + kb);
      int tot;
      const int slot = block_compact<NT>(j >= 0, L.wsum, &tot);
      if (j >= 0) L.tiles[slot] = 4 * j + 2 * (kb == rb.beta + 1) + (kb >= rb.beta);
      __syncthreads();
      wk.run(PairSetT<NS>{L.tiles, tot, wave});
      __syncthreads();
    }
  }
  __syncthreads();
}

// NT threads; wave w consumes the tiles of key stream w % NS (with more
// waves than streams, the waves of a stream split its rows).
// bits: the block-diagonal bitmap, (longest segment's blocks + 31) / 32 words
// of dynamic LDS (qmajor_bits_bytes).
// PM = 0: one query block, any index.  PM = kPairBlocks: the workgroup owns
// query blocks rb (even) and rb + 1 of a block selection (one segment, no
// lists), walked as a pair.  (Per-row selections keep one query block per
// workgroup: on the MoBA gate's selection at N = 131072 pairs made the
// forward 173.6 ms against 90.0 and dQ 124 against 110.)
constexpr int kPairBlocks = 1;

template <int NS = 4, int PM = 0, int NT, int NCOL, class Worker>
__device__ __forceinline__ void qmajor_drive(const AttnParams& p, const RowBlock& rb, int list,
                                             QMajorLds<NT, NCOL>& L, uint32_t* bits, Worker& wk) {
  if constexpr (PM == kPairBlocks) {
    qmajor_drive_pair<NS>(p, rb, list, L, wk);
  } else {
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane((tid >> 6) % NS);
  const int sp0 = p.s_ptr[list];
  const int ns = p.s_ptr[list + 1] - sp0;

  // Bitmap of the selected block-diagonals, for the "already covered" test.
  const int nwords = (rb.nb_seg + 31) >> 5;
  for (int w = tid; w < nwords; w += NT) bits[w] = 0u;
  __syncthreads();
  for (int e = tid; e < ns; e += NT) {
    const int g = p.s_idx[sp0 + e];
    if (g >= 0 && g < rb.nb_seg) atomicOr(&bits[g >> 5], 1u << (g & 31));
  }
  __syncthreads();

  // Vertical list: its length below the causal limit and its first chunks
  // are fetched before the slash walk, so that their latency hides behind it.
  const int vc = p.vcnt[list];
  const int* vs = p.vsel + (size_t)list * p.vsel_stride;
  const int lim_pos = (rb.qb_glob + 1) * kBlock;
  // vlimit = number of entries < lim_pos (the list is ascending), found by an
  // NT-ary search: every round samples NT evenly spaced entries of [lo, hi)
  // at once, so two rounds of loads cover lists of up to NT^2 entries.
  int lo = 0, hi = vc;  // entries below lo are < lim_pos, from hi on >= lim_pos
  while (lo < hi) {
    const int S = (hi - lo + NT - 1) / NT;
    const int e = lo + tid * S;
    const bool lt = e < hi && vs[e] < lim_pos;
    int k;
    block_compact<NT>(lt, L.wsum, &k);  // the true flags form a prefix
    __syncthreads();                    // L.wsum is reused by the next round
    if (k == 0) {
      hi = lo;
    } else {
      const int nlo = lo + (k - 1) * S + 1;
      hi = min(lo + k * S, hi);
      lo = nlo;
    }
  }
  const int vlimit = lo;
  // R chunks of NT candidates per batch: at most R*NT + 63 gathered columns
  constexpr int R = NCOL / NT - 1;
  static_assert(R >= 1, "column batch too small");
  int mv[R];
  auto fetch = [&](int e0) {
#pragma unroll
    for (int c = 0; c < R; ++c) {
      const int e = e0 + c * NT + tid;
      mv[c] = e < vlimit ? vs[e] : 0;
    }
  };
  fetch(0);

  // Block selection (an alternative estimator's index, one segment): the
  // 64-key blocks kb <= beta whose 128-block the query block's 128-block
  // selected (the second half of the diagonal 128-block lies past every
  // row of the first half and is left out by kb <= beta).
  if (p.bmask) {
    const int bh = list;  // one segment: list = b * h_q + h
    for (int base = 0; base <= rb.beta; base += NT) {
      const int kb = base + tid;
      int j = -1;
      if (kb <= rb.beta && bmask_bit(p, bh, rb.beta >> 1, kb >> 1)) j = local_key_block(p, rb.a_blk + kb);
      int tot;
      const int slot = block_compact<NT>(j >= 0, L.wsum, &tot);
      if (j >= 0) L.tiles[slot] = 2 * j + (kb == rb.beta);
      __syncthreads();
      wk.run(SlashSetT<NS>{L.tiles, tot, wave});
      __syncthreads();
    }
  }

  // Per-row block selection (another estimator's index, one segment): the
  // 64-key blocks kb <= beta of the blocks any row of the query block
  // picked; a tile is flagged when some row did not pick its block.  The
  // rows' words sit in the column buffer, which this index leaves unused.
  if (p.rmask) {
    static_assert(NCOL >= kBlock, "row words fit the column buffer");
    uint32_t* rsel = reinterpret_cast<uint32_t*>(L.cols);
    if (tid < kBlock) rsel[tid] = p.rmask[(size_t)list * p.n_q + (size_t)rb.i_local * kBlock + tid];
    __syncthreads();
    uint32_t uni = 0u, all = ~0u;
    for (int r = 0; r < kBlock; ++r) {
      const uint32_t w = rsel[r];
      uni |= w;
      all &= w;
    }
    for (int base = 0; base <= rb.beta; base += NT) {
      const int kb = base + tid;
      const int bb = kb >> p.rm_shift;
      int j = -1;
      if (kb <= rb.beta && ((uni >> bb) & 1u)) j = local_key_block(p, rb.a_blk + kb);
      int tot;
      const int slot = block_compact<NT>(j >= 0, L.wsum, &tot);
      if (j >= 0) L.tiles[slot] = 4 * j + 2 * (((all >> bb) & 1u) == 0u) + (kb == rb.beta);
      __syncthreads();
      wk.run(MobaSetT<NS>{L.tiles, tot, wave, rsel, p.rm_shift});
      __syncthreads();
    }
  }

  // Slash tiles: key block beta - g for every selected g <= beta.
  for (int base = 0; base < ns; base += NT) {
    const int e = base + tid;
    int j = -1, diag = 0;
    if (e < ns) {
      const int g = p.s_idx[sp0 + e];
      if (g >= 0 && g <= rb.beta) {
        j = local_key_block(p, rb.a_blk + rb.beta - g);
        diag = (g == 0);
      }
    }
    int tot;
    const int slot = block_compact<NT>(j >= 0, L.wsum, &tot);
    if (j >= 0) L.tiles[slot] = 2 * j + diag;
    __syncthreads();
    wk.run(SlashSetT<NS>{L.tiles, tot, wave});
    __syncthreads();
  }

  // Column tiles: verticals m < 64*(qb+1) not covered by a selected block,
  // gathered R chunks at a time; the next R chunks are fetched while the
  // current batch is walked.
  int count = 0, e0 = 0;
  while (e0 < vlimit) {
#pragma unroll
    for (int c = 0; c < R; ++c) {
      if (e0 + c * NT >= vlimit) break;  // uniform
      const int e = e0 + c * NT + tid;
      bool keep = false;
      const int m = mv[c];
      const int bm = m / kBlock - rb.a_blk;
      if (e < vlimit) {
        const int off = rb.beta - bm;
        keep = ((bits[off >> 5] >> (off & 31)) & 1u) == 0u;
      }
      int tot;
      const int slot = block_compact<NT>(keep, L.wsum, &tot);
      if (keep) {
        L.cols[count + slot] = local_key_pos(p, m);
        L.coff[count + slot] = (bm == rb.beta) ? (m - rb.qb_glob * kBlock) : -1;
      }
      count += tot;
      __syncthreads();
    }
    e0 += R * NT;
    const bool last = e0 >= vlimit;
    if (!last) fetch(e0);
    const int nt = last ? (count + 63) / 64 : count / 64;
    if (last && (count & 63) != 0) {
      // pad the last tile with a listed column that no row sees
      for (int t = count + tid; t < 64 * nt; t += NT) {
        L.cols[t] = L.cols[0];
        L.coff[t] = kBlock;
      }
      __syncthreads();
    }
    wk.run(ColSetT<NS>{L.cols, L.coff, last ? count : 64 * nt, nt, wave});
    if (last) break;
    __syncthreads();
    const int rem = count - 64 * nt;
    if (tid < rem) {
      L.cols[tid] = L.cols[64 * nt + tid];
      L.coff[tid] = L.coff[64 * nt + tid];
    }
    count = rem;
    __syncthreads();
  }
  __syncthreads();
  }
}

// Work-item mapping of a query-major grid of batch*h_q*nqb workgroups.  The
// dispatcher deals consecutive workgroup ids round-robin to the 8 XCDs, each
// with its own L2, and the mapping decides which tiles meet in an L2:
//   * by head (the default): each XCD takes batch*h_q/8 heads and walks all
//     their query blocks from the last (most keys) to the first, so
//     consecutive query blocks of a head run together and share its column
//     tiles and the tiles of nearby block-diagonals;
//   * by group (qmajor_item_units, when the index says the Q heads of a
//     (batch, KV head) group share most of their block-diagonals): every head
//     of a group on the same XCD, the heads of one query block in
//     consecutive slots, so they share the tiles of common diagonals; with
//     fewer groups than XCDs a group spreads over 8 / groups XCDs, which take
//     its query blocks in turn (block r goes to the group's XCD
//     r % (8 / groups), balancing the longer late blocks); with more, each
//     XCD takes whole groups.
// upg work units per group (its Q heads, or pairs of them); *unit = group *
// upg + unit in the group.
__device__ __forceinline__ void qmajor_item_units(const AttnParams& p, int wg, int upg, int nq, int* unit,
                                                  int* i_local) {
  const int NG = p.batch * p.h_kv;
  const int xcd = wg & 7;
  const int slot = wg >> 3;
  int ir;
  if (8 % NG == 0 && nq % (8 / NG) == 0) {
    const int xpg = 8 / NG;            // XCDs per group
    *unit = (xcd / xpg) * upg + slot % upg;
    ir = (slot / upg) * xpg + xcd % xpg;
  } else if (NG % 8 == 0) {
    const int per = NG / 8;            // groups per XCD
    const int u = slot % (per * upg);
    *unit = (xcd * per + u / upg) * upg + u % upg;
    ir = slot / (per * upg);
  } else {
    const int HB = NG * upg;
    *unit = wg % HB;
    ir = wg / HB;
  }
  *i_local = nq - 1 - ir;
}

// One Q head per workgroup: *hb = b * h_q + h, *i_local one of nq row items
// (the query blocks, or pairs of them).
__device__ __forceinline__ void qmajor_item(const AttnParams& p, int wg, int nq, int* hb, int* i_local) {
  if (p.map_group && *p.map_group) {
    qmajor_item_units(p, wg, p.h_q / p.h_kv, nq, hb, i_local);
    return;
  }
  const int HB = p.batch * p.h_q;
  int ir;
  if (HB % 8 == 0) {
    const int per = HB / 8;
    const int xcd = wg & 7;
    const int slot = wg >> 3;
    *hb = xcd * per + slot % per;
    ir = slot / per;
  } else {
    *hb = wg % HB;
    ir = wg / HB;
  }
  *i_local = nq - 1 - ir;
}

// Longest segment of a call, in blocks (the whole index grid when striped).
inline int max_segment_blocks(const AttnParams& p) {
  if (p.W != 1) return p.n_global / kBlock;
  int nb = 0;
  for (int s = 0; s < p.seg.n_seg; ++s) {
    const int l = p.seg.start_blk[s + 1] - p.seg.start_blk[s];
    nb = l > nb ? l : nb;
  }
  return nb;
}

// Dynamic LDS of the query-major kernels: the block-diagonal bitmap.
inline size_t qmajor_bits_bytes(const AttnParams& p) {
  return (size_t)((max_segment_blocks(p) + 31) / 32) * 4 + 4;
}

extern __shared__ uint32_t qm_bits[];

}  // namespace vs
