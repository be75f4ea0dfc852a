// vs_xattn_params.h — argument block of the XAttention block estimator.
#pragma once

#include "vs_attn_common.h"

namespace vs {

struct XaParams {
  const __bf16* q;
  const __bf16* k;
  Stride3 sq, sk;
  int batch, h_q, h_kv, n;  // n tokens per batch row (one segment)
  int nC, nI, words;        // cells, query blocks, bitmap words per row
  float sl2;                // scale * log2(e)
  float* cell_lse;          // [batch, h_q, nI, nC] log2-domain LSE of (key block, cell row)
  float threshold;
  uint32_t* bmask;          // [batch, h_q, nI, words]
  int* counts;              // [batch, h_q, nI] or null
  float* scores;            // [batch, h_q, nI, nI] or null
};

}  // namespace vs
