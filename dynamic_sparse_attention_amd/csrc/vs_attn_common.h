// vs_attn_common.h — argument block and tile descriptors shared by the sparse
// attention forward and backward kernels.
//
// The Vertical-Slash support of a query block (MTraining paper note,
// Algorithm 1, sparseformat; MTraining §4.1 (ii)-(iii)):
//   * slash tiles: for each selected block-diagonal g, the key block
//     beta - g of the same segment, if this call holds it (a causal mask
//     applies only when g == 0);
//   * column tiles: the selected vertical columns m <= the block's last row
//     whose block offset beta - beta(m) is not selected (those entries are
//     already inside a slash tile), 64 columns per tile, causal per row.
// Positions in the index are global (index coordinates); a block-striped
// call relabels global key block k_rank + W*j to local block j, or, holding
// every rank's chunk one after the other, global block u + W*j to local
// block u*(nkb/W) + j.
#pragma once

#include "vs_device.h"

namespace vs {

// Element strides of one [batch, token, head, channel] tensor (channels
// contiguous).
struct Stride3 {
  long long b, t, h;
  __host__ __device__ __forceinline__ long long at(long long bb, long long tt, long long hh) const {
    return bb * b + tt * t + hh * h;
  }
};

struct AttnParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;      // forward: output; backward: saved output (delta only)
  const void* dout;   // backward only
  const int* s_ptr;
  const int* s_idx;
  const int* vsel;    // prepared vertical lists: global positions held by this call
  const int* vcnt;
  int vsel_stride;
  void* o_out;
  float* lse;         // forward: written; backward: read
  const float* delta; // backward only
  const float* lse2;  // backward only: LSE * log2(e), +inf for an empty row
  float* delta_out;   // backward, bf16 dQ kernel: compute delta of its rows from o, dout and store it here
  float* lse2_out;    // backward, bf16 dQ kernel: store LSE * log2(e) of its rows here
  float* dq;
  float* dk;
  float* dv;
  int o_f32;
  int o_merge;        // forward: o_out (fp32) and lse hold a running result; merge this call's into them
  int* map_group;     // query-major grids: set on the device to 1 when the Q heads of a group share
                      // most of their block-diagonals (the group-wise work mapping), else 0; may be null
  int dq_accumulate;
  int batch, h_q, h_kv, n_q, n_k, nqb, nkb;
  float scale;
  float sl2;          // scale * log2(e)
  int W, q_rank, k_rank;
  int k_all;          // striped: K/V hold every rank's chunk (k_rank unused)
  int n_global;
  Stride3 sq, sk, sv, so, sdo;  // element strides of Q, K, V, O (its own type), dO
  // Block selection in place of the Vertical-Slash lists (one segment, W = 1):
  // bit J of row (b * h_q + h) * bm_nI + I marks 128-key block J for the
  // 128-row query block I; each 128-block covers two 64-blocks.
  const uint32_t* bmask;
  int bm_nI, bm_words;
  // Per-row block selection (MoBA's gate; one segment, batch-major rows):
  // bit J of rmask[(b * h_q + h) * n_q + n] marks key block J (of
  // 64 << rm_shift tokens) for row n; rm_union[(b * h_q + h) * nqb + i] is
  // the OR of the 64 rows' words of query block i (backward only).
  const uint32_t* rmask;
  const uint32_t* rm_union;
  int rm_shift;
  int qranges;        // backward column units: query-block ranges per column tile
  int qrange_len;
  int col_tiles;      // backward column units: column tiles per list
  int hh_lo, hh_hi;   // backward slash dK/dV: Q heads (within the GQA group) of this launch
  int kv_accumulate;  // backward slash dK/dV: add to dK/dV instead of storing
  int kv_parts;       // backward slash dK/dV: workgroups per key block, each over
                      // 1/kv_parts of the heads, adding with fp32 atomics when > 1
  SegTable seg;
};

// Global block of local query block i, and its segment / in-segment block.
struct RowBlock {
  int i_local;
  int qb_glob;
  int seg;
  int a_blk;   // segment start, in blocks
  int beta;    // block index inside the segment
  int nb_seg;  // blocks in the segment
};

__device__ __forceinline__ RowBlock row_block(const AttnParams& p, int i_local) {
  RowBlock rb;
  rb.i_local = i_local;
  if (p.W == 1) {
    rb.seg = seg_of_block(p.seg, i_local);
    rb.a_blk = p.seg.start_blk[rb.seg];
    rb.qb_glob = i_local;
    rb.nb_seg = p.seg.start_blk[rb.seg + 1] - rb.a_blk;
  } else {
    rb.seg = 0;
    rb.a_blk = 0;
    rb.qb_glob = p.q_rank + p.W * i_local;
    rb.nb_seg = p.n_global / kBlock;
  }
  rb.beta = rb.qb_glob - rb.a_blk;
  return rb;
}

// Local key block of global key block kb_glob, or -1 if this call does not hold it.
__device__ __forceinline__ int local_key_block(const AttnParams& p, int kb_glob) {
  if (p.W == 1) return (kb_glob >= 0 && kb_glob < p.nkb) ? kb_glob : -1;
  if (kb_glob < 0) return -1;
  if (p.k_all) {
    const int nc = p.nkb / p.W;  // key blocks per chunk
    const int j = kb_glob / p.W;
    return j < nc ? (kb_glob % p.W) * nc + j : -1;
  }
  const int d = kb_glob - p.k_rank;
  if (d < 0 || d % p.W != 0) return -1;
  const int j = d / p.W;
  return j < p.nkb ? j : -1;
}

// Global key block of local key block j (0 <= j < nkb).
__device__ __forceinline__ int global_key_block(const AttnParams& p, int j) {
  if (p.W == 1) return j;
  if (p.k_all) {
    const int nc = p.nkb / p.W;
    return j / nc + p.W * (j % nc);
  }
  return p.k_rank + p.W * j;
}

// Local query block of global block qb_glob, or -1 if this call does not hold it.
__device__ __forceinline__ int local_query_block(const AttnParams& p, int qb_glob) {
  if (p.W == 1) return (qb_glob >= 0 && qb_glob < p.nqb) ? qb_glob : -1;
  const int d = qb_glob - p.q_rank;
  if (d < 0 || d % p.W != 0) return -1;
  const int i = d / p.W;
  return i < p.nqb ? i : -1;
}

// Whether the block selection marks 128-key block J for 128-row block I of
// list bh (= b * h_q + h).
__device__ __forceinline__ bool bmask_bit(const AttnParams& p, int bh, int I, int J) {
  const uint32_t w = p.bmask[((size_t)bh * p.bm_nI + I) * p.bm_words + (J >> 5)];
  return (w >> (J & 31)) & 1u;
}

// Local key position of a global position held by this call.
__device__ __forceinline__ int local_key_pos(const AttnParams& p, int m_glob) {
  if (p.W == 1) return m_glob;
  return local_key_block(p, m_glob / kBlock) * kBlock + (m_glob % kBlock);
}

}  // namespace vs
