// vs_rows.h — K / V tiles of the row-split query-major kernels (bf16).
//
// The two waves of a key stream own query rows 0-31 and 32-63 of the block
// and share every 32-key tile of the stream: each issues half of the tile's
// direct global -> LDS loads (1 KiB per instruction, no registers), a
// workgroup barrier publishes both halves.  Operands are read from the tile in two ways:
//   * row reads (k_frag, ds_read_b128): the A operand of a product with the
//     tile's rows as output rows (S^T = K Q^T, dP^T = V dO^T), rows permuted
//     by slot_perm so that the result registers are the k slots of the next
//     product's B operand;
//   * transposed reads (t_frag, ds_read_b64_tr_b16): the A operand of a
//     product contracting over the tile's keys (O^T += V^T P^T,
//     dQ^T += K^T dS^T).
// gfx950's LDS serves 256 bytes per cycle: sixteen lanes of a 16-byte read or
// 32 lanes of an 8-byte read, so each such group must touch sixteen distinct
// 16-byte bank groups.  The layout that achieves it for both kinds of read:
// the rows of one direct load (RPI = 4 rows of 256 bytes for d = 128, 8 of
// 128 bytes for d = 64) are contiguous, each such 1 KiB group is followed by
// 16 bytes of padding (so successive groups start one bank group further
// on), and inside the group the 16-byte chunk c of row b sits at chunk index
// c ^ swz(b).  For d = 128, swz(b) = 4b puts the four rows of a group in four
// different quarters of the bank window (transposed reads take four
// consecutive rows) while the padding spreads the sixteen rows of a row read
// over the window; d = 64 uses swz(b) = 4 bit1(b) + 2 bit2(b) with two rows
// per window.  Per-lane offsets are computed once; the per-read part is an
// immediate.
#pragma once

#include "vs_qmajor.h"

namespace vs {

template <int D>
struct RowsTiles {
  typedef Mfma<__bf16> MF;
  typedef MF::frag frag;
  static constexpr int KPL = MF::KPL;
  static constexpr int KC = 2 * KPL;
  static constexpr int NCD = D / KC;   // k chunks over head_dim
  static constexpr int NCT = D / 32;   // 32-channel output tiles
  static constexpr int NCK = 32 / KC;  // k chunks over 32 keys
  static constexpr int CPR = D / 8;    // 16-byte chunks per row
  static constexpr int RPI = 64 / CPR; // rows per 1 KiB direct load
  static constexpr int NVL = 32 / RPI; // direct loads per 32-row tile
  static constexpr int GROUP = 1024 + 16;      // bytes per direct-load group, padded
  static constexpr int TB = NVL * GROUP;       // bytes per 32-row tile
  // chunk index XOR of row b (0 .. RPI-1) of a group
  __device__ static constexpr int swz(int b) {
    return D == 128 ? 4 * (b & 3) : 4 * ((b >> 1) & 1) + 2 * ((b >> 2) & 1);
  }

  int ro[4];
  int to[4];
  const __bf16* kb;   // K of (batch, kv head): key row pos at byte pos * krb
  const __bf16* vb;   // V of (batch, kv head): key row pos at byte pos * vrb
  uint32_t krb, vrb;  // row strides in bytes
  int rh;             // 32-row slice of this wave: 0-1 of one query block, 0-3 of a pair

  __device__ __forceinline__ void init_offsets() {
    const int lane = threadIdx.x & 63;
    const int hl = lane >> 5;
    // row operand: row sp, chunk 2c + hl
    const int sp = slot_perm<KPL>(lane & 31);
    const int a = sp / RPI, b = sp % RPI;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (D == 128) ro[j] = a * GROUP + b * 256 + 16 * hl + 64 * (j ^ b);  // j = c / 2
      else ro[j] = a * GROUP + b * 128 + 16 * hl + 32 * (j ^ (swz(b) >> 1));         // j = c
    }
    // transposed operand: lane i of a 16-lane group reads row 16c + 8h + 4q +
    // i/4 at chunk 4ct + x (x < 4), bytes 8 (i % 2) .. +7
    const int g = lane >> 4;
    const int sg = lane & 15;
    const int rr = sg >> 2;
    const int x = 2 * (g & 1) + ((sg & 3) >> 1);
    const int half = 8 * (sg & 1);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (D == 128) {
        to[j] = 2 * hl * GROUP + rr * 256 + 64 * (j ^ rr) + 16 * x + half;  // j = ct
      } else {
        const int ct = j >> 1, q = j & 1;                                   // j = 2 ct + q
        to[j] = hl * GROUP + (4 * q + rr) * 128 + 64 * (ct ^ ((rr >> 1) & 1)) + 16 * (x ^ (2 * q)) + half;
      }
    }
  }

  // Part `part` (wave-uniform, 0 .. NP-1) of the NVL direct loads of the 32
  // rows (K or V, from src) of half n into the tile at LDS address dst: load
  // u lands in group u, lane L at byte 16 L of it, i.e. row u * RPI + L / CPR,
  // chunk slot L % CPR, which holds chunk (L % CPR) ^ swz(L / CPR) of that
  // row.  dst is wave-uniform, so the LDS destinations stay in scalar
  // registers.  Byte offsets are 32-bit: the caller guarantees that
  // (n_k - 1) * rb + 256 < 2^32 for row stride rb (bytes).
  template <int NP, class Set>
  __device__ __forceinline__ void dma_part(const Set& S, int n, const __bf16* src, uint32_t rb, uint32_t dst,
                                           int part) const {
    constexpr int NU = NVL / NP;
    static_assert(NU >= 1 && NVL % NP == 0, "loads per part");
    const int lane = threadIdx.x & 63;
    const int rr = lane / CPR;
    const uint32_t cbyte = (uint32_t)(((lane % CPR) ^ swz(rr)) * 16);
    if constexpr (Set::kContiguous) {
      // consecutive rows: a wave-uniform base per load, the lane part fixed
      const int key0 = __builtin_amdgcn_readfirstlane(S.key_pos(n, part * NU * RPI));
      const char* g = reinterpret_cast<const char*>(src) + (size_t)key0 * rb;
      const uint32_t loff = (uint32_t)rr * rb + cbyte;
#pragma unroll
      for (int u0 = 0; u0 < NU; ++u0)
        dma_lds16_so(g + (size_t)(u0 * RPI) * rb, loff, dst + (part * NU + u0) * GROUP);
    } else {
      // gathered rows: every position is read from LDS before the first load
      // is issued, so the reads overlap
      uint32_t pos[NU];
#pragma unroll
      for (int u0 = 0; u0 < NU; ++u0) pos[u0] = (uint32_t)S.key_pos(n, (part * NU + u0) * RPI + rr);
#pragma unroll
      for (int u0 = 0; u0 < NU; ++u0)
        dma_lds16_so(src, pos[u0] * rb + cbyte, dst + (part * NU + u0) * GROUP);
    }
  }

  // This wave's share of the loads when the NP waves of a stream (the row
  // halves of one query block, or the row quarters of two) share them.
  template <int NP, class Set>
  __device__ __forceinline__ void dma_share(const Set& S, int n, const __bf16* src, uint32_t rb, uint32_t dst) const {
    dma_part<NP>(S, n, src, rb, dst, rh);
  }

  // Row operand: tile row slot_perm(L % 32), channels of k chunk c.
  __device__ __forceinline__ frag k_frag(const char* src, int c) const {
    if constexpr (D == 128) return *reinterpret_cast<const frag*>(src + ro[c >> 1] + 32 * (c & 1));
    else return *reinterpret_cast<const frag*>(src + ro[c]);
  }

  // Transposed operand: channels 32ct + L % 32, keys of k chunk c.
  // ds_read_b64_tr_b16: in each 16-lane group, lane i receives element i%4 of
  // the 8 bytes read by lanes i/4, 4+i/4, 8+i/4, 12+i/4, i.e. channel
  // 32ct + 16(g%2) + i of keys 16c + 8h + 4q .. +3.
  __device__ __forceinline__ frag t_frag(const char* src, int ct, int c) const {
    typedef short v4s __attribute__((ext_vector_type(4)));
    typedef short v8s __attribute__((ext_vector_type(8)));
    v4s part[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const char* a = D == 128 ? src + to[ct] + (4 * c + q) * GROUP : src + to[2 * ct + q] + 2 * c * GROUP;
      part[q] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)a);
    }
    const v8s both = __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(frag, both);
  }
};

// Index-expansion LDS for NS key streams: with one stream a workgroup (two
// waves) must fit in a quarter of the CU's LDS, so its column batches are
// smaller.
template <int NS> struct RowsLdsCfg {
  static constexpr int kCols = kColBatch;
};
template <> struct RowsLdsCfg<1> {
  static constexpr int kCols = 256;
};

}  // namespace vs
