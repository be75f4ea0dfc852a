// vs_qmajor.h — query-major walk over the Vertical-Slash support of one
// query block, shared by the forward kernel and the dQ backward kernel.
//
// A workgroup of 4 waves owns one (batch, Q head, query block).  It expands
// the index of the block on the fly (MTraining paper note, Algorithm 1
// sparseformat and Algorithm 2 convert_index): first the selected
// block-diagonals become key-block tiles, then the selected vertical columns
// that are not inside a selected block become 64-column tiles.  The tiles are
// dealt round-robin to the waves; each wave keeps its own running state for
// all 64 rows and the workgroup combines the four states at the end.
#pragma once

#include "vs_attn_common.h"

namespace vs {

constexpr int kQThreads = 256;
constexpr int kMaxBitWords = 2048;  // block offsets < 65536 (segments up to 4M tokens)

struct QMajorLds {
  uint32_t bits[kMaxBitWords];
  int tiles[kQThreads];
  int cols[2 * kQThreads];
  int coff[2 * kQThreads];
  int wsum[kQThreads / 64];
};

template <class Worker>
__device__ void qmajor_drive(const AttnParams& p, const RowBlock& rb, int list, QMajorLds& L,
                             Worker& wk) {
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  constexpr int NW = kQThreads / 64;
  const int sp0 = p.s_ptr[list];
  const int ns = p.s_ptr[list + 1] - sp0;

  // Bitmap of the selected block-diagonals, for the "already covered" test.
  const int nwords = (rb.nb_seg + 31) >> 5;
  for (int w = tid; w < nwords; w += kQThreads) L.bits[w] = 0u;
  __syncthreads();
  for (int e = tid; e < ns; e += kQThreads) {
    const int g = p.s_idx[sp0 + e];
    if (g >= 0 && g < rb.nb_seg) atomicOr(&L.bits[g >> 5], 1u << (g & 31));
  }
  __syncthreads();

  // Slash tiles: key block beta - g for every selected g <= beta.
  for (int base = 0; base < ns; base += kQThreads) {
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
    const int slot = block_compact<kQThreads>(j >= 0, L.wsum, &tot);
    if (j >= 0) L.tiles[slot] = 2 * j + diag;
    __syncthreads();
    for (int t = wave; t < tot; t += NW) {
      const int v = L.tiles[t];
      wk.tile(SlashTile{v >> 1, (v & 1) != 0});
    }
    __syncthreads();
  }

  // Column tiles: verticals m < 64*(qb+1) not covered by a selected block.
  const int vc = p.vcnt[list];
  const int* vs = p.vsel + (size_t)list * p.vsel_stride;
  const int lim_pos = (rb.qb_glob + 1) * kBlock;
  int lo = 0, hi = vc;  // first entry >= lim_pos
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (vs[mid] < lim_pos) lo = mid + 1; else hi = mid;
  }
  const int vlimit = lo;
  int count = 0, e0 = 0;
  while (true) {
    while (count < kQThreads && e0 < vlimit) {
      const int e = e0 + tid;
      bool keep = false;
      int m = 0, bm = 0;
      if (e < vlimit) {
        m = vs[e];
        bm = m / kBlock - rb.a_blk;
        const int off = rb.beta - bm;
        keep = ((L.bits[off >> 5] >> (off & 31)) & 1u) == 0u;
      }
      int tot;
      const int slot = block_compact<kQThreads>(keep, L.wsum, &tot);
      if (keep) {
        L.cols[count + slot] = local_key_pos(p, m);
        L.coff[count + slot] = (bm == rb.beta) ? (m - rb.qb_glob * kBlock) : -1;
      }
      count += tot;
      e0 += kQThreads;
      __syncthreads();
    }
    const bool last = e0 >= vlimit;
    const int nt = last ? (count + 63) / 64 : count / 64;
    for (int t = wave; t < nt; t += NW) {
      const int nc = count - 64 * t < 64 ? count - 64 * t : 64;
      wk.tile(ColTile{&L.cols[64 * t], &L.coff[64 * t], nc});
    }
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

// Work-item mapping of a query-major grid of batch*h_q*nqb workgroups.  The
// dispatcher deals consecutive workgroup ids round-robin to the 8 XCDs; the
// mapping gives each XCD a fixed set of heads (adjacent heads share a KV
// head) and walks its query blocks from the last (most keys) to the first, so
// blocks that share key blocks run close together on one L2.
__device__ __forceinline__ void qmajor_item(const AttnParams& p, int wg, int* hb, int* i_local) {
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
  *i_local = p.nqb - 1 - ir;
}

}  // namespace vs
