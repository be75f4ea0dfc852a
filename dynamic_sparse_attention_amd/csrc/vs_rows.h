// vs_rows.h — K / V tiles of the row-split query-major kernels (bf16).
//
// A workgroup of four waves serves two key streams; the two waves of a stream
// own query rows 0-31 and 32-63 of the block and share every 32-key tile of
// the stream: each issues half of the tile's direct global -> LDS loads
// (1 KiB per instruction, no registers), a workgroup barrier publishes both
// halves.  A tile is row-major (row r at r * D * 2 bytes) with the 16-byte
// chunk c of row r at chunk index c ^ swz(r), swz(r) = 2 (r mod 4) +
// floor(r / 8) mod 2, so that both kinds of operand read hit eight distinct
// bank groups:
//   * row reads (k_frag): the A operand of a product with the tile's rows as
//     output rows (S^T = K Q^T, dP^T = V dO^T), rows permuted by slot_perm so
//     that the result registers are the k slots of the next product's B
//     operand;
//   * transposed reads (t_frag, ds_read_b64_tr_b16): the A operand of a
//     product contracting over the tile's keys (O^T += V^T P^T,
//     dQ^T += K^T dS^T).
// Per-lane offsets are computed once; the per-read part is an immediate.
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
  static constexpr int NVH = NVL / 2;  // ... issued by each wave of a stream
  static constexpr int TB = 32 * D * 2;
  __device__ static constexpr int swz(int r) { return 2 * (r & 3) + ((r >> 3) & 1); }

  int ro[4];
  int to[2];
  const __bf16* kb;   // K of (batch, kv head): row pos at kb + pos * kvs
  const __bf16* vb;
  int kvs;
  int rh;             // row half of this wave

  __device__ __forceinline__ void init_offsets() {
    const int lane = threadIdx.x & 63;
    const int hl = lane >> 5;
    // row operand: row sp, chunk 2c + hl; the XOR permutes chunks inside
    // groups of 8, so the offset is ro[c % 4] + 128 * (c / 4)
    const int sp = slot_perm<KPL>(lane & 31);
#pragma unroll
    for (int cl = 0; cl < 4; ++cl) ro[cl] = sp * (CPR * 16) + 16 * ((2 * cl + hl) ^ swz(sp));
    // transposed operand: lane i of a 16-lane group reads row 16c + 8h + 4q +
    // i/4 at chunk 4ct + x (x < 4); swz = 2(i/4) + h, so the chunk is
    // 4 (ct ^ zh) + zl with z = x ^ swz
    const int g = lane >> 4;
    const int sg = lane & 15;
    const int rr = sg >> 2;
    const int x = 2 * (g & 1) + ((sg & 3) >> 1);
    const int z = x ^ (2 * rr + hl);
    const int base = (8 * hl + rr) * (CPR * 16) + 16 * (z & 3) + 8 * (sg & 1);
    to[0] = base + 64 * (z >> 2);
    to[1] = base + 64 * (1 - (z >> 2));
  }

  // This wave's half of the direct loads of the 32 rows (K or V, from src) of
  // half n into the tile at LDS address dst.
  template <class Set>
  __device__ __forceinline__ void dma_half(const Set& S, int n, const __bf16* src, uint32_t dst) const {
    const int lane = threadIdx.x & 63;
    const int rr = lane / CPR;
    const uint32_t rb = (uint32_t)(kvs * 2);
    if constexpr (Set::kContiguous) {
      const uint32_t o0 = (uint32_t)S.key_pos(n, rh * NVH * RPI + rr) * rb;
#pragma unroll
      for (int u0 = 0; u0 < NVH; ++u0) {
        const int u = rh * NVH + u0;
        const int chunk = (lane % CPR) ^ swz(u * RPI + rr);
        dma_lds16_so(src, o0 + (uint32_t)(u0 * RPI) * rb + chunk * 16, dst + u * 1024);
      }
    } else {
#pragma unroll
      for (int u0 = 0; u0 < NVH; ++u0) {
        const int u = rh * NVH + u0;
        const int chunk = (lane % CPR) ^ swz(u * RPI + rr);
        dma_lds16_so(src, (uint32_t)S.key_pos(n, u * RPI + rr) * rb + chunk * 16, dst + u * 1024);
      }
    }
  }

  // Row operand: tile row slot_perm(L % 32), channels of k chunk c.
  __device__ __forceinline__ frag k_frag(const char* src, int c) const {
    return *reinterpret_cast<const frag*>(src + ro[c & 3] + 128 * (c >> 2));
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
    for (int q = 0; q < 2; ++q)
      part[q] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(
          src + to[ct & 1] + 64 * (ct & ~1) + (16 * c + 4 * q) * (CPR * 16)));
    const v8s both = __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(frag, both);
  }
};

// Bitmap words of the row-split kernels: segments of up to 32768 blocks
// (longer ones take the four-wave kernels).
constexpr int kRowsBitWords = 1024;

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

}  // namespace vs
