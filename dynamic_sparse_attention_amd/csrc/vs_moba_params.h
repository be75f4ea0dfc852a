// vs_moba_params.h — argument block of the MoBA block gate.
#pragma once

#include "vs_attn_common.h"

namespace vs {

struct MobaParams {
  const __bf16* q;
  const __bf16* k;
  Stride3 sq, sk;
  int batch, h_q, h_kv, n, d;  // n tokens per batch row (one segment)
  int blk;                     // tokens per key block
  int nB;                      // key blocks (<= 32)
  int topk;
  float* kbar;                 // [batch, h_kv, nB, d] fp32: the blocks' mean keys
  uint32_t* rmask;             // [batch, h_q, n]: picked blocks per row
  float* scores;               // [batch, h_q, n, nB] or null
};

}  // namespace vs
