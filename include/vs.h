/*
 * vs.h — C ABI of the Vertical-Slash dynamic sparse attention library for
 * AMD Instinct MI355X (gfx950).
 *
 * The method is MTraining's dynamic sparse attention (MTraining, arXiv
 * 2510.18830, §3.2 and §4.1; the MTraining paper note, Algorithm 1 and
 * Algorithm 2): an online estimator scores the last query block against all
 * keys, keeps the top-k vertical key columns and the top-k slash
 * block-diagonals of the 64x64 block grid, and causal attention forward and
 * backward then run over that support only.  Partial results over successive
 * KV chunks combine with lse_merge.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every call validates all host-visible arguments before it enqueues
 *   anything; on error it returns a negative vs_status, enqueues nothing and
 *   records a message readable with vs_last_error().  No call allocates or
 *   frees device memory, and no call synchronises the stream: work is
 *   enqueued on the caller's hipStream_t (NULL = the default stream).
 * - Device buffers are caller-owned and must stay valid until the enqueued
 *   work completes.  Host arrays (vs_problem.cu_seqlens, budgets) are read
 *   only during the call.
 * - Tensor layout is [batch, token, head, head_dim] ("BSHD") for Q, K, V,
 *   O, dO, dQ, dK, dV and contiguous [batch, head, token] for LSE and delta.
 *   Q, K, V, O and dO take element strides for (batch, token, head) in
 *   vs_problem (head_dim contiguous), so that for instance slices of a fused
 *   QKV projection are passed without a copy; dQ, dK, dV, LSE and delta are
 *   contiguous.  Element types: Q, K, V, dO in vs_problem.dtype; O in that
 *   dtype or fp32 (o_f32); LSE, delta, dQ, dK, dV are fp32.
 * - LSE is the natural-log log-sum-exp of the scaled scores of a row over its
 *   support.  A row with an empty support has O = 0 and LSE = -inf and
 *   contributes no gradient.
 * - The index is a constant for the backward pass (the estimator is not
 *   differentiated), as in Algorithm 1 where the index is built from the
 *   observation window before the sparse attention call.
 */
#ifndef VS_H_
#define VS_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* vs_stream_t; /* the same object as hipStream_t */

typedef int32_t vs_status;
enum {
  VS_OK = 0,
  VS_ERR_NULL = -1,        /* a required pointer is NULL                               */
  VS_ERR_SHAPE = -2,       /* inconsistent sizes, heads, segments or stripes           */
  VS_ERR_UNSUPPORTED = -3, /* valid request outside what the GPU path implements       */
  VS_ERR_BUDGET = -4,      /* negative budget                                          */
  VS_ERR_WORKSPACE = -5,   /* workspace smaller than vs_workspace_size()               */
  VS_ERR_HIP = -6,         /* a HIP launch failed; vs_last_error() has its message     */
  VS_ERR_INDEX = -7        /* index capacities inconsistent with the problem           */
};

typedef enum { VS_F32 = 0, VS_BF16 = 1 } vs_dtype;

/* Which rows and keys one call holds, in the coordinates of the index.
 *
 * Index coordinates are token positions 0..n_global-1 of one batch row,
 * n_global = cu_seqlens[n_seg].  Segments [cu_seqlens[s], cu_seqlens[s+1])
 * are packed documents: attention never crosses a segment boundary and each
 * segment has its own index.  Inside a segment starting at a, the block of
 * position p is beta(p) = (p - a) / block.
 *
 * Contiguous layout (stripe_world == 1): the call holds every row and key,
 * n_q == n_k == n_global.
 * Block-striped layout (stripe_world = W > 1, one segment only; MTraining
 * §4.2 (ii): 64-token stripes): local row block i is global block
 * q_rank + W*i and local key block j is global block k_rank + W*j, so
 * n_global == W*n_q == W*n_k.  A striped call computes the global mask
 * restricted to its rows and keys; one worker's ring step on KV chunk u is
 * the call with q_rank = worker, k_rank = u.
 * All chunks at once (k_rank = VS_ALL_CHUNKS): K and V hold the W chunks one
 * after the other, chunk u (the keys of rank u) at rows u*n_global/W ..
 * (u+1)*n_global/W - 1, so n_k == n_global; local key block u*(n_k/W) + j is
 * global block u + W*j.  The call is the whole ring of one worker (every step
 * of Algorithm 2's inner loop) in one pass: the rows' softmax runs over all
 * chunks at once, so no partial result is merged, and dK / dV come out for
 * every chunk, in the same chunk-after-chunk layout.
 *
 * Strides: x_stride[0..2] are the element strides of batch, token and head
 * (head_dim is contiguous).  All three zero selects the contiguous layout
 * ([batch, n, heads, head_dim] with n = n_q for Q, O, dO and n_k for K, V).
 * Otherwise each must be >= 0 and a multiple of 8 elements, and the tensor's
 * base pointer 16-byte aligned; rows of the output O must not overlap.
 * o_stride is in elements of O's type (fp32 when o_f32).  For bf16 inputs
 * the kernels address the rows of one (batch, KV head) of K and V with
 * 32-bit byte offsets: (n_k - 1) * token stride * 2 + 256 must stay below
 * 2^32 (else VS_ERR_UNSUPPORTED).
 */
typedef struct vs_problem {
  int32_t batch;        /* >= 1                                                   */
  int32_t h_q;          /* query heads, a multiple of h_kv                         */
  int32_t h_kv;         /* key/value heads; Q head h reads KV head h*h_kv/h_q      */
  int32_t head_dim;     /* 64 or 128                                              */
  int32_t n_q;          /* rows per batch row held by this call                   */
  int32_t n_k;          /* keys per batch row held by this call (bf16: see the
                           32-bit offset limit under Strides above)               */
  int32_t block;        /* B, 64 (the slash granularity of MTraining §4.1 (ii))    */
  int32_t dtype;        /* vs_dtype of Q, K, V, dO (and O unless o_f32)            */
  float scale;          /* score scale; <= 0 selects 1/sqrt(head_dim)             */
  int32_t n_seg;        /* 1..VS_MAX_SEGMENTS segments per batch row               */
  const int32_t* cu_seqlens; /* HOST, n_seg+1 ascending token offsets, [0]=0;
                                every segment length a multiple of block (>0) */
  int32_t stripe_world; /* 1 = contiguous, W > 1 = block-striped                   */
  int32_t q_rank;       /* striped: rank whose row blocks this call holds          */
  int32_t k_rank;       /* striped: rank whose key blocks this call holds, or
                           VS_ALL_CHUNKS: K/V hold every rank's chunk              */
  int64_t q_stride[3];  /* element strides (batch, token, head); all 0 = contiguous */
  int64_t k_stride[3];
  int64_t v_stride[3];
  int64_t o_stride[3];  /* of O, in O's element type                              */
  int64_t do_stride[3]; /* of dO                                                  */
} vs_problem;

#define VS_MAX_SEGMENTS 128
#define VS_ALL_CHUNKS (-1)

/* The Vertical-Slash index, one list pair per (batch b, Q head h, segment s),
 * list number l = (b*h_q + h)*n_seg + s.  All four arrays are DEVICE memory.
 * v_idx[v_ptr[l] .. v_ptr[l+1]) are the selected vertical key columns as
 * index-coordinate token positions inside segment s, strictly ascending;
 * s_idx[s_ptr[l] .. s_ptr[l+1]) are the selected block-diagonal offsets
 * g = beta(row) - beta(key) >= 0, strictly ascending.  Entries < 0 (padding
 * written by vs_estimate_index when a capacity exceeds the candidates) are
 * ignored.  v_cap_max / s_cap_max are HOST-known upper bounds of the list
 * lengths (vs_index_capacity returns them) used to size launches.
 *
 * Block selection (an alternative estimator's index, vs_estimate_index_xattn):
 * when blk_mask is not NULL the index is a selection of blk_size x blk_size
 * blocks instead of Vertical-Slash lists: row n attends key m iff m <= n and
 * bit J = m / blk_size of word J / 32 of row
 * (b * h_q + h) * nI + n / blk_size is set, nI = ceil(n_global / blk_size),
 * ceil(nI / 32) words per row (DEVICE).  It requires bf16 inputs, one
 * segment, stripe_world 1, blk_size 128 and empty lists (v_cap_max and
 * s_cap_max 0; v_ptr and s_ptr still point at batch*h_q+1 zero offsets),
 * else VS_ERR_UNSUPPORTED / VS_ERR_INDEX.
 *
 * Per-row block selection (another estimator's index, vs_estimate_index_moba):
 * when row_mask is not NULL, row n of (b, h) attends key m iff m <= n and bit
 * J = m / row_blk of the word row_mask[(b * h_q + h) * n_global + n] is set
 * (DEVICE, one 32-bit word per row).  It requires bf16 inputs, one segment,
 * stripe_world 1, row_blk a power of two >= 64 with n_global <= 32 * row_blk,
 * empty lists as for blk_mask, and blk_mask NULL, else VS_ERR_UNSUPPORTED /
 * VS_ERR_INDEX.
 */
typedef struct vs_index {
  const int32_t* v_ptr;
  const int32_t* v_idx;
  const int32_t* s_ptr;
  const int32_t* s_idx;
  int32_t v_cap_max;
  int32_t s_cap_max;
  const uint32_t* blk_mask;  /* NULL: the Vertical-Slash lists above */
  int32_t blk_size;
  const uint32_t* row_mask;  /* NULL: no per-row block selection */
  int32_t row_blk;
} vs_index;

/* List offsets for budgets (MTraining paper note, Algorithm 1: argtopk with
 * budgets k_v and k_s; MTraining §4.1 (ii): verticals per token, slashes per
 * 64x64 block-diagonal).  v_budget[h], s_budget[h] (HOST, h_q entries) are
 * tokens for the whole batch row.  Segment s of length L receives
 * ceil(k*L/n_global) of each; the vertical share is clipped to L columns and
 * the slash share becomes min(ceil(share/block), ceil(L/block))
 * block-diagonals.  Writes v_ptr_host / s_ptr_host (HOST, batch*h_q*n_seg+1
 * entries each) and, when not NULL, the largest list lengths.
 * Errors: VS_ERR_NULL, VS_ERR_SHAPE, VS_ERR_BUDGET (a budget < 0). */
vs_status vs_index_capacity(const vs_problem* p, const int32_t* v_budget,
                            const int32_t* s_budget, int32_t* v_ptr_host,
                            int32_t* s_ptr_host, int32_t* v_cap_max,
                            int32_t* s_cap_max);

/* Workspace bytes an entry point needs: op 0 = vs_estimate_index (and
 * vs_estimate_index_topp),
 * 1 = vs_sparse_attn_fwd, 2 = vs_sparse_attn_bwd, 3 = vs_estimate_index_xattn,
 * 4 = vs_estimate_index_moba.  idx may be NULL for op 0;
 * for ops 1 and 2 it supplies the capacity bounds.  The workspace is DEVICE
 * memory, 256-byte aligned, owned by the caller, and may be reused across
 * calls on the same stream. */
vs_status vs_workspace_size(const vs_problem* p, int32_t op, const vs_index* idx,
                            size_t* bytes);

/* Online index estimation (MTraining paper note, Algorithm 1, first six
 * steps; MTraining §4.1 (i)-(ii)).  For every (b, h, s): the last block of
 * segment s (last_q = block rows) is the observation window; each window
 * row r gets a causal softmax A_hat[r, m] over the segment's keys m <= r;
 * the vertical score of column m is sum_r A_hat[r, m] and the slash score of
 * block-diagonal g is the window mass on it; the v_ptr/s_ptr capacities of
 * the highest scores are kept (ties to the lowest index) and written
 * ascending into v_idx / s_idx (padding -1 when a capacity exceeds the
 * candidates).  Scores are computed from bf16/fp32 inputs with fp32
 * accumulation.
 * q: [batch, n, h_q, d]; k: [batch, n, h_kv, d] (DEVICE, strides from the
 * problem; the estimation sees the whole sequence: stripe_world must be 1).  v_ptr, s_ptr: DEVICE offsets from
 * vs_index_capacity.  v_score [batch, h_q, n] and s_score
 * [batch, h_q, n/block] (fp32, DEVICE, nullable) receive the scores; s_score
 * entry of segment s, offset g, is at [b, h, cu_seqlens[s]/block + g].
 * last_q: 0 or block (other window sizes are VS_ERR_UNSUPPORTED).
 * Errors: VS_ERR_NULL, VS_ERR_SHAPE, VS_ERR_UNSUPPORTED, VS_ERR_WORKSPACE,
 * VS_ERR_HIP. */
vs_status vs_estimate_index(const vs_problem* p, const void* q, const void* k,
                            int32_t last_q, const int32_t* v_ptr, int32_t* v_idx,
                            const int32_t* s_ptr, int32_t* s_idx, float* v_score,
                            float* s_score, void* ws, size_t ws_bytes,
                            vs_stream_t stream);

/* Online index estimation with top-p budgets (MTraining paper note,
 * Algorithm 1: k_v = topp(sum_v(A_hat), p_v), k_s = topp(pooled sum_s(A_hat),
 * p_s); MTraining §4.1 (i): the fewest lines that recall a target share of
 * the window's attention mass).  Scores as in vs_estimate_index; then for
 * every (b, h, s) and kind, k = the fewest highest scores (ties to the lowest
 * index) whose mass reaches the fraction p_v[h] (verticals) or p_s[h]
 * (block-diagonals) of the list's total, capped by the list's capacity
 * (v_ptr / s_ptr from vs_index_capacity, whose budgets act as upper bounds).
 * The k selected entries are written ascending at the start of the list and
 * the rest of its capacity is padded with -1.  The comparison is exact: a
 * score s has integer mass rint(s * 2^54), the target is
 * ceil(rint(p * 2^24) * total / 2^24), p clamped to [0, 1] (NaN as 0).
 * p_v, p_s: DEVICE fp32, h_q entries each.  counts (DEVICE, nullable):
 * receives k per list and kind at [2*l + 0] (verticals) and [2*l + 1]
 * (block-diagonals).  Workspace: op 0 of vs_workspace_size.  Other arguments
 * and errors as vs_estimate_index. */
vs_status vs_estimate_index_topp(const vs_problem* p, const void* q, const void* k,
                                 int32_t last_q, const float* p_v, const float* p_s,
                                 const int32_t* v_ptr, int32_t* v_idx, const int32_t* s_ptr,
                                 int32_t* s_idx, int32_t* counts, float* v_score,
                                 float* s_score, void* ws, size_t ws_bytes,
                                 vs_stream_t stream);

/* XAttention block estimation, an alternative index estimator for the same
 * attention calls (the MTraining paper note, appendix, baseline settings,
 * item 2: blocks scored by sums along their anti-diagonals sampled at a
 * stride, the high-scoring ones kept; block 128, stride 16, threshold 0.9).
 * For every (b, h): cell logits z[A, C] = (1/stride) sum_u scale *
 * q[stride A + u] . k[stride C + stride - 1 - u] (u < stride) for cells
 * C <= A; a softmax over each cell row; block scores s[I, J] = the sum of
 * the probabilities of the block's cells; for each query block I the fewest
 * key blocks J <= I, highest scores first (ties to the lowest J), whose
 * integer masses rint(s * 2^50) reach ceil(rint(t * 2^24) * total / 2^24)
 * (t = threshold clamped to [0, 1]).  Writes blk_mask (DEVICE, the layout of
 * vs_index.blk_mask) and, when not NULL, counts [b, h_q, nI] int32 (blocks
 * kept) and blk_score [b, h_q, nI, nI] fp32 (s; entries J > I unspecified).
 * q [batch, n, h_q, d], k [batch, n, h_kv, d] bf16 (strides from the
 * problem); one segment, stripe_world 1, block 128, stride 16 and n at most
 * 131072 (1024 query blocks), else VS_ERR_UNSUPPORTED.  Workspace: op 3.
 * Errors: VS_ERR_NULL, VS_ERR_SHAPE, VS_ERR_UNSUPPORTED, VS_ERR_WORKSPACE,
 * VS_ERR_HIP. */
vs_status vs_estimate_index_xattn(const vs_problem* p, const void* q, const void* k,
                                  int32_t block, int32_t stride, float threshold,
                                  uint32_t* blk_mask, int32_t* counts, float* blk_score,
                                  void* ws, size_t ws_bytes, vs_stream_t stream);

/* MoBA block gate, a second alternative estimator for the same attention
 * calls (the MTraining paper note, appendix, baseline settings, item 1: key
 * blocks of fixed size, a per-query MoE-style gate picking the top-k blocks,
 * the query's own block always among them; block 4096, top-12).  For every
 * (b, h): the mean kbar_J of each key block J of `block` tokens (the last may
 * be short); for every row n the gate scores q_n . kbar_J (fp32) of the
 * blocks J before its own block n / block; the picked set is the own block
 * and the topk - 1 highest-scoring earlier blocks, ties to the lowest J (all
 * earlier blocks when there are fewer).  Writes row_mask (DEVICE, the layout
 * of vs_index.row_mask) and, when not NULL, gate_scores [b, h_q, n, nB] fp32
 * (nB = ceil(n / block); entries of the own block and later unspecified).
 * q [batch, n, h_q, d], k [batch, n, h_kv, d] bf16 (strides from the
 * problem); one segment, stripe_world 1, block a power of two >= 256 with
 * n <= 32 * block, topk >= 1, else VS_ERR_UNSUPPORTED / VS_ERR_SHAPE.
 * Workspace: op 4.  Errors: VS_ERR_NULL, VS_ERR_SHAPE, VS_ERR_UNSUPPORTED,
 * VS_ERR_WORKSPACE, VS_ERR_HIP. */
vs_status vs_estimate_index_moba(const vs_problem* p, const void* q, const void* k, int32_t block,
                                 int32_t topk, uint32_t* row_mask, float* gate_scores, void* ws,
                                 size_t ws_bytes, vs_stream_t stream);

/* Sparse attention forward (MTraining paper note, Algorithm 1 last step and
 * Algorithm 2 block_bar_sparse_attention_forward; online softmax as in
 * "Ring Attention Paper Analysis", "The Blockwise Partitioning Strategy").
 * Row n attends to key m iff they share a segment, m <= n, and m is a
 * selected vertical or beta(n) - beta(m) a selected block-diagonal of the
 * row's (b, h, s) list.  q [batch, n_q, h_q, d], k/v [batch, n_k, h_kv, d]
 * (DEVICE, dtype).  o [batch, n_q, h_q, d] (fp32 if o_f32 else dtype),
 * lse [batch, h_q, n_q] fp32.  Rows are fully overwritten, except with
 * o_f32 = 2: then o (fp32) and lse hold a running result (O = 0, LSE = -inf
 * for nothing yet) and this call's result is merged into them in place, as
 * lse_merge does (merge_out_and_lse of Algorithm 2, fused: one ring step of a
 * striped worker without a partial buffer).  o_f32 other than 0, 1, 2 is
 * VS_ERR_SHAPE.
 * Errors: VS_ERR_NULL, VS_ERR_SHAPE, VS_ERR_UNSUPPORTED, VS_ERR_INDEX,
 * VS_ERR_WORKSPACE, VS_ERR_HIP. */
vs_status vs_sparse_attn_fwd(const vs_problem* p, const void* q, const void* k,
                             const void* v, const vs_index* idx, void* o, int32_t o_f32,
                             float* lse, void* ws, size_t ws_bytes, vs_stream_t stream);

/* delta[b, h, n] = sum_c dout[b, n, h, c] * o[b, n, h, c], the row term
 * rowsum(dA * A) of MTraining §3.2 Eq. 1 (it equals rowsum(dO * O)).
 * o is fp32 if o_f32 else dtype; dout is dtype; delta fp32 [batch, h_q, n_q].
 * Errors: VS_ERR_NULL, VS_ERR_SHAPE, VS_ERR_UNSUPPORTED, VS_ERR_HIP. */
vs_status vs_attn_bwd_delta(const vs_problem* p, const void* o, int32_t o_f32,
                            const void* dout, float* delta, vs_stream_t stream);

/* Sparse attention backward over the same support (MTraining §3.2 Eq. 1-2;
 * paper note Appendix B.1): P = exp(S - lse), dP = dO V^T,
 * dS = P * (dP - delta), dQ = scale dS K, dK = scale dS^T Q, dV = P^T dO,
 * dK and dV summed over the Q heads of a KV group.  lse and delta are the
 * FINAL values of the rows (after every KV chunk was merged); delta may be
 * NULL, then it is computed from o and dout into the workspace (o and dout
 * are read only in that case).  dq [batch, n_q, h_q, d] fp32 is overwritten,
 * or accumulated into when dq_accumulate != 0; dk, dv [batch, n_k, h_kv, d]
 * fp32 are overwritten.  With bf16 inputs a GQA group holds at most 32 Q
 * heads (h_q / h_kv <= 32), else VS_ERR_UNSUPPORTED.
 * Errors: VS_ERR_NULL, VS_ERR_SHAPE, VS_ERR_UNSUPPORTED, VS_ERR_INDEX,
 * VS_ERR_WORKSPACE, VS_ERR_HIP. */
vs_status vs_sparse_attn_bwd(const vs_problem* p, const void* q, const void* k,
                             const void* v, const void* o, int32_t o_f32,
                             const void* dout, const float* lse, const float* delta,
                             const vs_index* idx, float* dq, int32_t dq_accumulate,
                             float* dk, float* dv, void* ws, size_t ws_bytes,
                             vs_stream_t stream);

/* vs_sparse_attn_bwd without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving or
 * training loops, harnesses that forbid hipMalloc.  The workspace is a fixed
 * array of VS_NOALLOC_SCRATCH_BYTES bytes inside the library, one per GPU,
 * placed there when the library's kernels are loaded on the device and held
 * until the process ends; the call allocates and frees nothing.  Its device
 * address is looked up on the first call on each device.  Arguments, results
 * and errors are those of vs_sparse_attn_bwd; a problem whose backward
 * workspace (vs_workspace_size, op 2) exceeds the array returns
 * VS_ERR_WORKSPACE before any HIP call.  Every call on one GPU uses the same
 * array and leaves it in an unspecified state (each call writes every part it
 * reads before reading it): calls whose work may overlap on one GPU (on
 * different streams, or on different host threads) race on it and must be
 * serialised by the caller. */
#define VS_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
vs_status vs_sparse_attn_bwd_noalloc(const vs_problem* p, const void* q, const void* k,
                                     const void* v, const void* o, int32_t o_f32,
                                     const void* dout, const float* lse, const float* delta,
                                     const vs_index* idx, float* dq, int32_t dq_accumulate,
                                     float* dk, float* dv, vs_stream_t stream);

/* merge_out_and_lse (MTraining paper note, Algorithm 2): combine a partial
 * result over a disjoint key set into an accumulator, in place:
 * L = max(l1, l2) + log(e^(l1-max) + e^(l2-max)),
 * O = e^(l1-L) O1 + e^(l2-L) O2, where a partial with LSE = -inf is the
 * identity and two empty partials stay (O = 0, LSE = -inf).
 * o_acc, o_part: fp32 [batch, n, heads, head_dim]; lse_acc, lse_part: fp32
 * [batch, heads, n] (DEVICE).  head_dim a power of two from 4 to 256.
 * Errors: VS_ERR_NULL, VS_ERR_SHAPE, VS_ERR_UNSUPPORTED, VS_ERR_HIP. */
vs_status lse_merge(int32_t batch, int32_t n, int32_t heads, int32_t head_dim,
                    float* o_acc, float* lse_acc, const float* o_part,
                    const float* lse_part, vs_stream_t stream);

/* Per-kernel timing, a profiling aid.  While enabled, every kernel the library
 * launches is bracketed by two HIP events on its stream (the launch itself is
 * unchanged).  vs_trace_collect waits for the recorded events and writes one
 * line per kernel name, "name launches total_ms\n", into buf (HOST,
 * NUL-terminated, truncated to len bytes), then forgets them.  Events are
 * created on first use and reused; tracing adds no device allocation.
 * Errors: VS_ERR_NULL (buf), VS_ERR_HIP (an event failed). */
vs_status vs_trace_enable(int32_t on);
vs_status vs_trace_collect(char* buf, size_t len);

/* Message for the last non-OK status returned on the calling thread. */
const char* vs_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* VS_H_ */
