// vs_stage.h — transposed staging of row-major tiles into LDS.
//
// The matrix cores take the k dimension contiguous per lane.  For products
// that contract over tokens (P V, dS K, P^T dO, dS^T Q) the token dimension
// must be contiguous, but K, V, Q and dO are stored token-major.  These
// helpers read NROWS rows with 16-byte global loads and write them
// channel-major into LDS with 8-byte stores (KG tokens of one channel each).
#pragma once

#include "vs_device.h"

namespace vs {

// dst[ch * P + r] = row r of the tile, channel ch, for r < NROWS, ch < D.
// pos(r) gives the row's element offset in global memory (row start).
template <typename T, int D, int NROWS, int P, int NT, class PosF>
__device__ __forceinline__ void stage_transposed(T* dst, const T* base, PosF pos, int t) {
  constexpr int CG = 16 / (int)sizeof(T);
  constexpr int KG = 8 / (int)sizeof(T);
  constexpr int NRG = NROWS / KG;
  constexpr int NGRP = NRG * (D / CG);
#pragma unroll
  for (int g0 = 0; g0 < NGRP; g0 += NT) {
    const int g = g0 + t;
    if (NGRP % NT != 0 && g >= NGRP) break;
    const int rg = g % NRG;
    const int cg = g / NRG;
    T vals[KG][CG];
#pragma unroll
    for (int u = 0; u < KG; ++u)
      *reinterpret_cast<f32x4*>(&vals[u][0]) =
          *reinterpret_cast<const f32x4*>(base + pos(rg * KG + u) + cg * CG);
#pragma unroll
    for (int c = 0; c < CG; ++c) {
      T pk[KG];
#pragma unroll
      for (int u = 0; u < KG; ++u) pk[u] = vals[u][c];
      *reinterpret_cast<f32x2*>(dst + (cg * CG + c) * P + rg * KG) = *reinterpret_cast<const f32x2*>(pk);
    }
  }
}

}  // namespace vs
