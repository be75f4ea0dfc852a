// vs_api.cpp — the C ABI: argument validation, workspace layout and launches.
//
// Every entry point validates all host-visible arguments before the first
// HIP call, so a rejected call enqueues nothing (and needs no GPU).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/vs.h"
#include "vs_attn_common.h"
#include "vs_trace.h"

namespace vs {
hipError_t launch_fwd(const AttnParams& p, int dtype_bf16, int d, hipStream_t st);
hipError_t launch_prep_vertical(const AttnParams& p, int n_lists, const int* v_ptr, const int* v_idx,
                                hipStream_t st);
hipError_t launch_delta(const void* o, Stride3 so, int o_f32, int bf16, const void* dout, Stride3 sdo,
                        float* delta, int batch, int n, int h, int d, hipStream_t st);
hipError_t launch_lse_log2(const float* lse, float* lse2, size_t count, hipStream_t st);
hipError_t launch_lse_merge(int batch, int n, int heads, int d, float* o_acc, float* lse_acc,
                            const float* o_part, const float* lse_part, hipStream_t st);
hipError_t launch_bwd(const AttnParams& p, int dtype_bf16, int d, hipStream_t st);
struct EstParams;
hipError_t launch_estimate(const AttnParams& p, int dtype_bf16, int d, const int* v_ptr, int* v_idx,
                           const int* s_ptr, int* s_idx, float* v_score, float* s_score,
                           float2* partials, float* lse2, int tiles_total, const int* tile_prefix,
                           const float* p_v, const float* p_s, int* kcount, uint2* cand, int* ccount,
                           hipStream_t st);
constexpr int kEstKeyTile = 256;
constexpr int kTopkChunk = 16384;  // entries per first-stage workgroup of a long vertical list
struct XaParams;
hipError_t launch_xattn(const XaParams& p, int d, hipStream_t st);
struct MobaParams;
hipError_t launch_moba(const MobaParams& p, hipStream_t st);
hipError_t launch_moba_union(const uint32_t* rmask, uint32_t* out, int tiles, hipStream_t st);
}  // namespace vs

#include "vs_xattn_params.h"
#include "vs_moba_params.h"

namespace {

thread_local std::string g_err;

vs_status fail(vs_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

vs_status ok() {
  g_err.clear();
  return VS_OK;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct Prob {
  int batch, h_q, h_kv, d, n_q, n_k, block, bf16, n_seg, W, q_rank, k_rank, k_all, n_global, nqb, nkb;
  float scale;
  std::vector<int> cu;
  vs::Stride3 sq, sk, sv, so, sdo;
  int n_lists() const { return batch * h_q * n_seg; }
};

// Element strides of one tensor: all zero selects the contiguous layout
// [batch, n, heads, d]; otherwise each must be >= 0 and a multiple of 8
// elements (16-byte loads of bf16 rows).
vs_status stride_of(const int64_t* in, long long n, long long heads, long long d, const char* name,
                    vs::Stride3* out) {
  if (in[0] == 0 && in[1] == 0 && in[2] == 0) {
    *out = {n * heads * d, heads * d, d};
    return VS_OK;
  }
  static const char* dim[3] = {"batch", "token", "head"};
  for (int i = 0; i < 3; ++i) {
    if (in[i] < 0) return fail(VS_ERR_SHAPE, "%s %s stride %lld is negative", name, dim[i], (long long)in[i]);
    if (in[i] % 8 != 0)
      return fail(VS_ERR_UNSUPPORTED, "%s %s stride %lld is not a multiple of 8 elements", name, dim[i],
                  (long long)in[i]);
  }
  *out = {in[0], in[1], in[2]};
  return VS_OK;
}

vs_status check_problem(const vs_problem* p, Prob* c) {
  if (!p) return fail(VS_ERR_NULL, "problem is NULL");
  if (!p->cu_seqlens) return fail(VS_ERR_NULL, "cu_seqlens is NULL");
  if (p->batch < 1 || p->h_q < 1 || p->h_kv < 1)
    return fail(VS_ERR_SHAPE, "batch, h_q, h_kv must be >= 1 (got %d, %d, %d)", p->batch, p->h_q,
                p->h_kv);
  if (p->h_q % p->h_kv != 0)
    return fail(VS_ERR_SHAPE, "h_q (%d) must be a multiple of h_kv (%d)", p->h_q, p->h_kv);
  if (p->head_dim != 64 && p->head_dim != 128)
    return fail(VS_ERR_UNSUPPORTED, "head_dim %d unsupported (64 or 128)", p->head_dim);
  if (p->block != 64) return fail(VS_ERR_UNSUPPORTED, "block %d unsupported (64)", p->block);
  if (p->dtype != VS_F32 && p->dtype != VS_BF16)
    return fail(VS_ERR_UNSUPPORTED, "dtype %d unsupported", p->dtype);
  if (p->n_seg < 1) return fail(VS_ERR_SHAPE, "n_seg must be >= 1 (got %d)", p->n_seg);
  if (p->n_seg > VS_MAX_SEGMENTS)
    return fail(VS_ERR_UNSUPPORTED, "n_seg %d exceeds %d", p->n_seg, VS_MAX_SEGMENTS);
  if (!(std::isfinite(p->scale))) return fail(VS_ERR_SHAPE, "scale is not finite");
  if (p->n_q < 0 || p->n_k < 0) return fail(VS_ERR_SHAPE, "n_q, n_k must be >= 0");
  c->cu.assign(p->cu_seqlens, p->cu_seqlens + p->n_seg + 1);
  if (c->cu[0] != 0) return fail(VS_ERR_SHAPE, "cu_seqlens[0] must be 0");
  for (int s = 0; s < p->n_seg; ++s) {
    const long long L = (long long)c->cu[s + 1] - c->cu[s];
    if (L <= 0) return fail(VS_ERR_SHAPE, "segment %d has length %lld", s, L);
    if (L % p->block != 0)
      return fail(VS_ERR_UNSUPPORTED, "segment %d length %lld is not a multiple of %d", s, L,
                  p->block);
    if (L / p->block > 65536)
      return fail(VS_ERR_UNSUPPORTED, "segment %d longer than 65536 blocks", s);
  }
  c->n_global = c->cu[p->n_seg];
  c->W = p->stripe_world;
  c->k_all = 0;
  if (c->W < 1) return fail(VS_ERR_SHAPE, "stripe_world must be >= 1");
  if (c->W == 1) {
    if (p->n_q != c->n_global || p->n_k != c->n_global)
      return fail(VS_ERR_SHAPE, "contiguous call needs n_q == n_k == cu_seqlens[n_seg] (%d, %d, %d)",
                  p->n_q, p->n_k, c->n_global);
  } else {
    if (p->n_seg != 1) return fail(VS_ERR_UNSUPPORTED, "striped calls take one segment");
    if (c->n_global % (p->block * c->W) != 0)
      return fail(VS_ERR_SHAPE, "n_global %d not a multiple of block*stripe_world", c->n_global);
    c->k_all = p->k_rank == VS_ALL_CHUNKS;
    const int nk_want = c->k_all ? c->n_global : c->n_global / c->W;
    if (p->n_q != c->n_global / c->W || p->n_k != nk_want)
      return fail(VS_ERR_SHAPE, "striped call needs n_q == n_global/stripe_world and n_k == %s",
                  c->k_all ? "n_global (all chunks)" : "n_global/stripe_world");
    if (p->q_rank < 0 || p->q_rank >= c->W || (!c->k_all && (p->k_rank < 0 || p->k_rank >= c->W)))
      return fail(VS_ERR_SHAPE, "q_rank/k_rank outside [0, stripe_world) (k_rank may be VS_ALL_CHUNKS)");
  }
  if ((long long)p->batch * p->n_q > (1ll << 31) / 64 || (long long)p->batch * p->n_k > (1ll << 31) / 64)
    return fail(VS_ERR_UNSUPPORTED, "batch * tokens too large");
  vs_status st;
  if ((st = stride_of(p->q_stride, p->n_q, p->h_q, p->head_dim, "q", &c->sq))) return st;
  if ((st = stride_of(p->k_stride, p->n_k, p->h_kv, p->head_dim, "k", &c->sk))) return st;
  if ((st = stride_of(p->v_stride, p->n_k, p->h_kv, p->head_dim, "v", &c->sv))) return st;
  if ((st = stride_of(p->o_stride, p->n_q, p->h_q, p->head_dim, "o", &c->so))) return st;
  if ((st = stride_of(p->do_stride, p->n_q, p->h_q, p->head_dim, "do", &c->sdo))) return st;
  // The bf16 attention kernels address the K and V rows of one (batch, KV
  // head) with 32-bit byte offsets from a per-(batch, head) base.
  if (p->dtype == VS_BF16 && p->n_k > 0) {
    const long long kmax = (long long)(p->n_k - 1) * c->sk.t * 2 + 256;
    const long long vmax = (long long)(p->n_k - 1) * c->sv.t * 2 + 256;
    if (kmax >= (1ll << 32) || vmax >= (1ll << 32))
      return fail(VS_ERR_UNSUPPORTED,
                  "K/V rows of one head span %lld / %lld bytes, beyond the kernels' 4 GiB offsets", kmax, vmax);
  }
  c->batch = p->batch;
  c->h_q = p->h_q;
  c->h_kv = p->h_kv;
  c->d = p->head_dim;
  c->n_q = p->n_q;
  c->n_k = p->n_k;
  c->block = p->block;
  c->bf16 = p->dtype == VS_BF16;
  c->n_seg = p->n_seg;
  c->q_rank = c->W == 1 ? 0 : p->q_rank;
  c->k_rank = c->W == 1 ? 0 : p->k_rank;
  c->nqb = p->n_q / p->block;
  c->nkb = p->n_k / p->block;
  c->scale = p->scale > 0.f ? p->scale : 1.0f / std::sqrt((float)p->head_dim);
  return VS_OK;
}

vs_status check_index(const Prob& c, const vs_index* idx) {
  if (!idx) return fail(VS_ERR_NULL, "index is NULL");
  if (!idx->v_ptr || !idx->s_ptr) return fail(VS_ERR_NULL, "index v_ptr/s_ptr is NULL");
  if (idx->v_cap_max < 0 || idx->s_cap_max < 0)
    return fail(VS_ERR_INDEX, "negative index capacity bound");
  if (idx->v_cap_max > 0 && !idx->v_idx) return fail(VS_ERR_NULL, "index v_idx is NULL");
  if (idx->s_cap_max > 0 && !idx->s_idx) return fail(VS_ERR_NULL, "index s_idx is NULL");
  int max_seg = 0;
  for (int s = 0; s < c.n_seg; ++s) max_seg = std::max(max_seg, c.cu[s + 1] - c.cu[s]);
  if (idx->v_cap_max > max_seg)
    return fail(VS_ERR_INDEX, "v_cap_max %d exceeds the longest segment %d", idx->v_cap_max, max_seg);
  if (idx->s_cap_max > max_seg / c.block)
    return fail(VS_ERR_INDEX, "s_cap_max %d exceeds the block count %d", idx->s_cap_max,
                max_seg / c.block);
  if (idx->row_mask) {
    if (!c.bf16 || c.W != 1 || c.n_seg != 1)
      return fail(VS_ERR_UNSUPPORTED, "a per-row block selection takes bf16 inputs, one segment, no striping");
    const int rb = idx->row_blk;
    if (rb < c.block || (rb & (rb - 1)) != 0)
      return fail(VS_ERR_UNSUPPORTED, "per-row selection blocks of %d tokens (a power of two >= %d)", rb, c.block);
    if ((int64_t)c.n_global > 32 * (int64_t)rb)
      return fail(VS_ERR_UNSUPPORTED, "a per-row selection holds 32 blocks per row (n %d, blocks of %d)",
                  c.n_global, rb);
    if (idx->blk_mask) return fail(VS_ERR_INDEX, "a block selection and a per-row selection together");
    if (idx->v_cap_max != 0 || idx->s_cap_max != 0)
      return fail(VS_ERR_INDEX, "a per-row selection comes with empty Vertical-Slash lists");
  }
  if (idx->blk_mask) {
    if (!c.bf16 || c.W != 1 || c.n_seg != 1)
      return fail(VS_ERR_UNSUPPORTED, "a block selection takes bf16 inputs, one segment, no striping");
    if (idx->blk_size != 2 * c.block)
      return fail(VS_ERR_UNSUPPORTED, "block selection of %d-token blocks unsupported (%d)", idx->blk_size,
                  2 * c.block);
    if (idx->v_cap_max != 0 || idx->s_cap_max != 0)
      return fail(VS_ERR_INDEX, "a block selection comes with empty Vertical-Slash lists");
  }
  return VS_OK;
}

// The block-selection fields of the kernels' argument block.
void fill_bmask(const Prob& c, const vs_index* idx, vs::AttnParams* a) {
  a->bmask = idx->blk_mask;
  if (idx->blk_mask) {
    a->bm_nI = (c.n_global + idx->blk_size - 1) / idx->blk_size;
    a->bm_words = (a->bm_nI + 31) / 32;
  }
  a->rmask = idx->row_mask;
  if (idx->row_mask) {
    int sh = 0;
    while ((c.block << sh) < idx->row_blk) ++sh;
    a->rm_shift = sh;  // row_blk = 64 << sh (checked a power of two)
  }
}

void fill_params(const Prob& c, vs::AttnParams* a) {
  std::memset(a, 0, sizeof *a);
  a->batch = c.batch;
  a->h_q = c.h_q;
  a->h_kv = c.h_kv;
  a->n_q = c.n_q;
  a->n_k = c.n_k;
  a->nqb = c.nqb;
  a->nkb = c.nkb;
  a->scale = c.scale;
  a->sl2 = c.scale * vs::kLog2e;
  a->W = c.W;
  a->q_rank = c.q_rank;
  a->k_rank = c.k_rank;
  a->k_all = c.k_all;
  a->n_global = c.n_global;
  a->sq = c.sq;
  a->sk = c.sk;
  a->sv = c.sv;
  a->so = c.so;
  a->sdo = c.sdo;
  a->seg.n_seg = c.n_seg;
  for (int s = 0; s <= c.n_seg; ++s) a->seg.start_blk[s] = c.cu[s] / c.block;
}

// Workspace layouts.
struct AttnWs {
  size_t vsel, vcnt, share, delta, lse2, rm_union, total;
};
// Forward: prepared vertical lists.  Backward: also delta (when the caller
// gives none) and LSE * log2(e), one fp32 per (batch, Q head, row) each, and
// with a per-row block selection the OR of each query block's rows' words.
AttnWs attn_ws(const Prob& c, const vs_index* idx, bool backward) {
  const int v_cap_max = idx->v_cap_max;
  AttnWs w;
  size_t off = 0;
  w.vsel = off;
  off += align256((size_t)c.n_lists() * std::max(v_cap_max, 1) * 4);
  w.vcnt = off;
  off += align256((size_t)c.n_lists() * 4);
  w.share = off;  // the work-mapping flag of the query-major kernels
  off += 256;
  const size_t rows = align256((size_t)c.batch * c.h_q * c.n_q * 4);
  w.delta = off;
  if (backward) off += rows;
  w.lse2 = off;
  if (backward) off += rows;
  w.rm_union = off;
  if (backward && idx->row_mask) off += align256((size_t)c.batch * c.h_q * c.nqb * 4);
  w.total = off;
  return w;
}

struct EstWs {
  size_t part, lse2, vscore, sscore, kcount, cand, ccount, tprefix, total;
  int tiles_total;
  int nchunk;  // top-k first-stage chunks per vertical list (< 2: none)
  std::vector<int> tile_prefix;
};
EstWs est_ws(const Prob& c) {
  EstWs w;
  w.tile_prefix.assign(c.n_seg + 1, 0);
  for (int s = 0; s < c.n_seg; ++s)
    w.tile_prefix[s + 1] =
        w.tile_prefix[s] + (c.cu[s + 1] - c.cu[s] + vs::kEstKeyTile - 1) / vs::kEstKeyTile;
  w.tiles_total = w.tile_prefix[c.n_seg];
  size_t off = 0;
  w.part = off;
  off += align256((size_t)c.batch * c.h_q * w.tiles_total * 64 * 8);
  w.lse2 = off;
  off += align256((size_t)c.n_lists() * 64 * 4);
  w.vscore = off;
  off += align256((size_t)c.batch * c.h_q * c.n_global * 4);
  w.sscore = off;
  off += align256((size_t)c.batch * c.h_q * (c.n_global / c.block) * 4);
  w.kcount = off;  // top-p: entries per (list, kind)
  off += align256((size_t)c.n_lists() * 2 * 4);
  // top-k of long vertical lists: each 16384-entry chunk's candidates
  // (score bits, index) and their number
  int max_len = 0;
  for (int s = 0; s < c.n_seg; ++s) max_len = std::max(max_len, c.cu[s + 1] - c.cu[s]);
  w.nchunk = (max_len + vs::kTopkChunk - 1) / vs::kTopkChunk;
  const size_t nc = w.nchunk >= 2 ? (size_t)c.n_lists() * w.nchunk : 0;
  w.cand = off;
  off += align256(nc * vs::kTopkChunk * 8);
  w.ccount = off;
  off += align256(nc * 4);
  w.tprefix = off;
  w.total = off;
  return w;
}

// XAttention estimate: per (batch, Q head) the log-sum-exp of every (key
// block, cell row) (fp32, log2 domain).
struct XaWs {
  size_t cell, total;
  int nC, nI;
};
// MoBA gate: the blocks' mean keys, [batch, h_kv, nB, d] fp32, for blocks of
// blk tokens (the 32-block maximum when blk is not yet known).
size_t moba_ws(const Prob& c, int blk) {
  const int nB = blk > 0 ? (c.n_global + blk - 1) / blk : 32;
  return align256((size_t)c.batch * c.h_kv * nB * c.d * 4);
}

XaWs xa_ws(const Prob& c) {
  XaWs w;
  w.nC = c.n_global / 16;
  w.nI = (c.n_global + 127) / 128;
  size_t off = 0;
  w.cell = off;
  off += align256((size_t)c.batch * c.h_q * w.nC * w.nI * 4);
  w.total = off;
  return w;
}

vs_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(VS_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

}  // namespace


// ---------------------------------------------------------------------------
// Per-kernel timing (vs_trace_enable / vs_trace_collect).
namespace {
struct TraceRec {
  const char* name;
  hipEvent_t start, stop;
};
std::mutex g_tmu;
bool g_trace = false;
std::vector<TraceRec> g_pending;
std::vector<hipEvent_t> g_pool;
thread_local hipEvent_t t_start = nullptr;
thread_local const char* t_name = nullptr;

hipEvent_t pool_event() {
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}
}  // namespace

namespace vs {
void trace_begin(hipStream_t st, const char* name) {
  std::lock_guard<std::mutex> lk(g_tmu);
  t_start = nullptr;
  if (!g_trace) return;
  t_start = pool_event();
  t_name = name;
  if (t_start) (void)hipEventRecord(t_start, st);
}
void trace_end(hipStream_t st) {
  std::lock_guard<std::mutex> lk(g_tmu);
  if (!g_trace || !t_start) return;
  hipEvent_t stop = pool_event();
  if (!stop) return;
  (void)hipEventRecord(stop, st);
  g_pending.push_back({t_name, t_start, stop});
  t_start = nullptr;
}
}  // namespace vs

extern "C" {

const char* vs_last_error(void) { return g_err.c_str(); }

vs_status vs_index_capacity(const vs_problem* p, const int32_t* v_budget, const int32_t* s_budget,
                            int32_t* v_ptr_host, int32_t* s_ptr_host, int32_t* v_cap_max,
                            int32_t* s_cap_max) {
  Prob c;
  vs_status st = check_problem(p, &c);
  if (st) return st;
  if (!v_budget || !s_budget || !v_ptr_host || !s_ptr_host)
    return fail(VS_ERR_NULL, "budget or pointer array is NULL");
  for (int h = 0; h < c.h_q; ++h)
    if (v_budget[h] < 0 || s_budget[h] < 0)
      return fail(VS_ERR_BUDGET, "head %d has a negative budget", h);
  long long vo = 0, so = 0;
  int vmax = 0, smax = 0;
  const long long N = c.n_global;
  v_ptr_host[0] = 0;
  s_ptr_host[0] = 0;
  for (int b = 0; b < c.batch; ++b)
    for (int h = 0; h < c.h_q; ++h)
      for (int s = 0; s < c.n_seg; ++s) {
        const long long L = c.cu[s + 1] - c.cu[s];
        const long long nb = (L + c.block - 1) / c.block;
        const long long sv = ((long long)v_budget[h] * L + N - 1) / N;
        const long long ss = ((long long)s_budget[h] * L + N - 1) / N;
        const long long kv = std::min(sv, L);
        const long long kg = std::min((ss + c.block - 1) / c.block, nb);
        vo += kv;
        so += kg;
        if (vo > INT32_MAX || so > INT32_MAX) return fail(VS_ERR_SHAPE, "index too large");
        const int l = (b * c.h_q + h) * c.n_seg + s;
        v_ptr_host[l + 1] = (int32_t)vo;
        s_ptr_host[l + 1] = (int32_t)so;
        vmax = std::max(vmax, (int)kv);
        smax = std::max(smax, (int)kg);
      }
  if (v_cap_max) *v_cap_max = vmax;
  if (s_cap_max) *s_cap_max = smax;
  return ok();
}

vs_status vs_workspace_size(const vs_problem* p, int32_t op, const vs_index* idx, size_t* bytes) {
  Prob c;
  vs_status st = check_problem(p, &c);
  if (st) return st;
  if (!bytes) return fail(VS_ERR_NULL, "bytes is NULL");
  if (op == 0) {
    *bytes = est_ws(c).total;
    return ok();
  }
  if (op == 3) {
    *bytes = xa_ws(c).total;
    return ok();
  }
  if (op == 4) {
    *bytes = moba_ws(c, 0);
    return ok();
  }
  if (op != 1 && op != 2) return fail(VS_ERR_SHAPE, "op %d is not 0, 1, 2, 3 or 4", op);
  if ((st = check_index(c, idx))) return st;
  *bytes = attn_ws(c, idx, op == 2).total;
  return ok();
}

namespace {
vs_status estimate(const char* what, const vs_problem* p, const void* q, const void* k, int32_t last_q,
                   const float* p_v, const float* p_s, const int32_t* v_ptr, int32_t* v_idx,
                   const int32_t* s_ptr, int32_t* s_idx, int32_t* counts, float* v_score,
                   float* s_score, void* ws, size_t ws_bytes, vs_stream_t stream) {
  Prob c;
  vs_status st = check_problem(p, &c);
  if (st) return st;
  if (c.W != 1) return fail(VS_ERR_UNSUPPORTED, "estimation runs on the contiguous layout");
  if (last_q != 0 && last_q != c.block)
    return fail(VS_ERR_UNSUPPORTED, "last_q %d unsupported (0 or %d)", last_q, c.block);
  if (!q || !k || !v_ptr || !s_ptr || !v_idx || !s_idx)
    return fail(VS_ERR_NULL, "q, k, v_ptr, v_idx, s_ptr or s_idx is NULL");
  const EstWs w = est_ws(c);
  if (!ws || ws_bytes < w.total)
    return fail(VS_ERR_WORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, w.total);
  vs::AttnParams a;
  fill_params(c, &a);
  a.q = q;
  a.k = k;
  char* base = static_cast<char*>(ws);
  float* vsc = v_score ? v_score : reinterpret_cast<float*>(base + w.vscore);
  float* ssc = s_score ? s_score : reinterpret_cast<float*>(base + w.sscore);
  int* kc = counts ? counts : reinterpret_cast<int*>(base + w.kcount);
  return hip_status(vs::launch_estimate(a, c.bf16, c.d, v_ptr, v_idx, s_ptr, s_idx, vsc, ssc,
                                        reinterpret_cast<float2*>(base + w.part),
                                        reinterpret_cast<float*>(base + w.lse2), w.tiles_total,
                                        w.tile_prefix.data(), p_v, p_s, kc,
                                        w.nchunk >= 2 ? reinterpret_cast<uint2*>(base + w.cand) : nullptr,
                                        w.nchunk >= 2 ? reinterpret_cast<int*>(base + w.ccount) : nullptr,
                                        (hipStream_t)stream),
                    what);
}
}  // namespace

vs_status vs_estimate_index(const vs_problem* p, const void* q, const void* k, int32_t last_q,
                            const int32_t* v_ptr, int32_t* v_idx, const int32_t* s_ptr,
                            int32_t* s_idx, float* v_score, float* s_score, void* ws,
                            size_t ws_bytes, vs_stream_t stream) {
  return estimate("vs_estimate_index", p, q, k, last_q, nullptr, nullptr, v_ptr, v_idx, s_ptr, s_idx,
                  nullptr, v_score, s_score, ws, ws_bytes, stream);
}

vs_status vs_estimate_index_topp(const vs_problem* p, const void* q, const void* k, int32_t last_q,
                                 const float* p_v, const float* p_s, const int32_t* v_ptr,
                                 int32_t* v_idx, const int32_t* s_ptr, int32_t* s_idx,
                                 int32_t* counts, float* v_score, float* s_score, void* ws,
                                 size_t ws_bytes, vs_stream_t stream) {
  if (!p_v || !p_s) return fail(VS_ERR_NULL, "p_v or p_s is NULL");
  return estimate("vs_estimate_index_topp", p, q, k, last_q, p_v, p_s, v_ptr, v_idx, s_ptr, s_idx,
                  counts, v_score, s_score, ws, ws_bytes, stream);
}

vs_status vs_estimate_index_xattn(const vs_problem* p, const void* q, const void* k, int32_t block,
                                  int32_t stride, float threshold, uint32_t* blk_mask, int32_t* counts,
                                  float* blk_score, void* ws, size_t ws_bytes, vs_stream_t stream) {
  Prob c;
  vs_status st = check_problem(p, &c);
  if (st) return st;
  if (!q || !k || !blk_mask) return fail(VS_ERR_NULL, "q, k or blk_mask is NULL");
  if (!c.bf16 || c.W != 1 || c.n_seg != 1)
    return fail(VS_ERR_UNSUPPORTED, "XAttention estimation takes bf16 inputs, one segment, no striping");
  if (block != 128 || stride != 16)
    return fail(VS_ERR_UNSUPPORTED, "XAttention block %d / stride %d unsupported (128 / 16)", block, stride);
  if (c.n_global > 131072)
    return fail(VS_ERR_UNSUPPORTED, "XAttention estimation sorts at most 1024 key blocks (n %d)", c.n_global);
  if (!std::isfinite(threshold)) return fail(VS_ERR_SHAPE, "threshold is not finite");
  const XaWs w = xa_ws(c);
  if (!ws || ws_bytes < w.total)
    return fail(VS_ERR_WORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, w.total);
  vs::XaParams x;
  std::memset(&x, 0, sizeof x);
  x.q = static_cast<const __bf16*>(q);
  x.k = static_cast<const __bf16*>(k);
  x.sq = c.sq;
  x.sk = c.sk;
  x.batch = c.batch;
  x.h_q = c.h_q;
  x.h_kv = c.h_kv;
  x.n = c.n_global;
  x.nC = w.nC;
  x.nI = w.nI;
  x.words = (w.nI + 31) / 32;
  x.sl2 = c.scale * vs::kLog2e;
  char* base = static_cast<char*>(ws);
  x.cell_lse = reinterpret_cast<float*>(base + w.cell);
  x.threshold = threshold;
  x.bmask = blk_mask;
  x.counts = counts;
  x.scores = blk_score;
  return hip_status(vs::launch_xattn(x, c.d, (hipStream_t)stream), "vs_estimate_index_xattn");
}

vs_status vs_estimate_index_moba(const vs_problem* p, const void* q, const void* k, int32_t block,
                                 int32_t topk, uint32_t* row_mask, float* gate_scores, void* ws,
                                 size_t ws_bytes, vs_stream_t stream) {
  Prob c;
  vs_status st = check_problem(p, &c);
  if (st) return st;
  if (!q || !k || !row_mask) return fail(VS_ERR_NULL, "q, k or row_mask is NULL");
  if (!c.bf16 || c.W != 1 || c.n_seg != 1)
    return fail(VS_ERR_UNSUPPORTED, "MoBA estimation takes bf16 inputs, one segment, no striping");
  if (block < 256 || (block & (block - 1)) != 0)
    return fail(VS_ERR_UNSUPPORTED, "MoBA block %d unsupported (a power of two >= 256)", block);
  if ((int64_t)c.n_global > 32 * (int64_t)block)
    return fail(VS_ERR_UNSUPPORTED, "MoBA estimation picks among at most 32 blocks (n %d, block %d)", c.n_global,
                block);
  if (topk < 1) return fail(VS_ERR_SHAPE, "topk %d < 1", topk);
  const size_t need = moba_ws(c, block);
  if (!ws || ws_bytes < need) return fail(VS_ERR_WORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, need);
  vs::MobaParams m;
  std::memset(&m, 0, sizeof m);
  m.q = static_cast<const __bf16*>(q);
  m.k = static_cast<const __bf16*>(k);
  m.sq = c.sq;
  m.sk = c.sk;
  m.batch = c.batch;
  m.h_q = c.h_q;
  m.h_kv = c.h_kv;
  m.n = c.n_global;
  m.d = c.d;
  m.blk = block;
  m.nB = (c.n_global + block - 1) / block;
  m.topk = topk;
  m.kbar = static_cast<float*>(ws);
  m.rmask = row_mask;
  m.scores = gate_scores;
  return hip_status(vs::launch_moba(m, (hipStream_t)stream), "vs_estimate_index_moba");
}

vs_status vs_sparse_attn_fwd(const vs_problem* p, const void* q, const void* k, const void* v,
                             const vs_index* idx, void* o, int32_t o_f32, float* lse, void* ws,
                             size_t ws_bytes, vs_stream_t stream) {
  Prob c;
  vs_status st = check_problem(p, &c);
  if (st) return st;
  if ((st = check_index(c, idx))) return st;
  if (!q || !k || !v || !o || !lse) return fail(VS_ERR_NULL, "q, k, v, o or lse is NULL");
  const AttnWs w = attn_ws(c, idx, false);
  if (!ws || ws_bytes < w.total)
    return fail(VS_ERR_WORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, w.total);
  vs::AttnParams a;
  fill_params(c, &a);
  a.q = q;
  a.k = k;
  a.v = v;
  a.s_ptr = idx->s_ptr;
  a.s_idx = idx->s_idx;
  fill_bmask(c, idx, &a);
  char* base = static_cast<char*>(ws);
  a.vsel = reinterpret_cast<int*>(base + w.vsel);
  a.vcnt = reinterpret_cast<int*>(base + w.vcnt);
  a.map_group = reinterpret_cast<int*>(base + w.share);
  a.vsel_stride = std::max(idx->v_cap_max, 1);
  if (o_f32 < 0 || o_f32 > 2) return fail(VS_ERR_SHAPE, "o_f32 %d is not 0, 1 or 2", o_f32);
  a.o_out = o;
  a.o_f32 = o_f32 != 0;
  a.o_merge = o_f32 == 2;
  a.lse = lse;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = vs::launch_prep_vertical(a, c.n_lists(), idx->v_ptr, idx->v_idx, s);
  if (e == hipSuccess) e = vs::launch_fwd(a, c.bf16, c.d, s);
  return hip_status(e, "vs_sparse_attn_fwd");
}

vs_status vs_attn_bwd_delta(const vs_problem* p, const void* o, int32_t o_f32, const void* dout,
                            float* delta, vs_stream_t stream) {
  Prob c;
  vs_status st = check_problem(p, &c);
  if (st) return st;
  if (!o || !dout || !delta) return fail(VS_ERR_NULL, "o, dout or delta is NULL");
  return hip_status(vs::launch_delta(o, c.so, o_f32 != 0, c.bf16, dout, c.sdo, delta, c.batch, c.n_q,
                                     c.h_q, c.d, (hipStream_t)stream),
                    "vs_attn_bwd_delta");
}

}  // extern "C"

// Workspace of vs_sparse_attn_bwd_noalloc: a file-scope device array, one
// copy per GPU (placed there when the library's code object is loaded on the
// device, and held until the process ends).  Host code never passes the
// array's name to a kernel: it is a host-side stand-in, so its device address
// is looked up once per device and kept in g_scratch_ptr.
static __device__ __align__(256) char scratch[VS_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the device of `stream` (the current
// device for the null stream), looked up on the first call for that device
// with the device current.
vs_status scratch_of(hipStream_t stream, void** out) {
  int cur = -1, dev = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return fail(VS_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  dev = cur;
  if (stream) {
    e = hipStreamGetDevice(stream, &dev);
    if (e != hipSuccess) return fail(VS_ERR_HIP, "hipStreamGetDevice: %s", hipGetErrorString(e));
  }
  if (dev < 0 || dev >= kMaxDevices) return fail(VS_ERR_UNSUPPORTED, "device %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess)
      return fail(VS_ERR_HIP, "hipSetDevice(%d): %s", dev, hipGetErrorString(e));
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (dev != cur) (void)hipSetDevice(cur);
    if (e != hipSuccess || !ptr)
      return fail(VS_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return VS_OK;
}

// The backward; with ws == NULL and use_scratch, the workspace is the
// device's scratch array (sizes beyond it are refused before any HIP call).
vs_status attn_bwd(const char* what, const vs_problem* p, const void* q, const void* k, const void* v,
                   const void* o, int32_t o_f32, const void* dout, const float* lse, const float* delta,
                   const vs_index* idx, float* dq, int32_t dq_accumulate, float* dk, float* dv, void* ws,
                   size_t ws_bytes, bool use_scratch, vs_stream_t stream) {
  Prob c;
  vs_status st = check_problem(p, &c);
  if (st) return st;
  if ((st = check_index(c, idx))) return st;
  if (!q || !k || !v || !dout || !lse || !dq || !dk || !dv)
    return fail(VS_ERR_NULL, "q, k, v, dout, lse, dq, dk or dv is NULL");
  if (!delta && !o) return fail(VS_ERR_NULL, "o is NULL and no delta was given");
  // The bf16 dK/dV kernels tag each staged query tile with the Q head's
  // index inside its GQA group in the top bits of a 32-bit word (0 .. 31).
  if (c.bf16 && c.h_q / c.h_kv > 32)
    return fail(VS_ERR_UNSUPPORTED, "bf16 backward takes at most 32 Q heads per KV head (got %d)",
                c.h_q / c.h_kv);
  const AttnWs w = attn_ws(c, idx, true);
  if (use_scratch) {
    if (w.total > VS_NOALLOC_SCRATCH_BYTES)
      return fail(VS_ERR_WORKSPACE, "%s: the problem needs %zu bytes of workspace, beyond the library's "
                  "fixed %zu bytes", what, w.total, (size_t)VS_NOALLOC_SCRATCH_BYTES);
    if ((st = scratch_of((hipStream_t)stream, &ws))) return st;
    ws_bytes = VS_NOALLOC_SCRATCH_BYTES;
  }
  if (!ws || ws_bytes < w.total)
    return fail(VS_ERR_WORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, w.total);
  vs::AttnParams a;
  fill_params(c, &a);
  a.q = q;
  a.k = k;
  a.v = v;
  a.dout = dout;
  a.s_ptr = idx->s_ptr;
  a.s_idx = idx->s_idx;
  fill_bmask(c, idx, &a);
  char* base = static_cast<char*>(ws);
  a.vsel = reinterpret_cast<int*>(base + w.vsel);
  a.vcnt = reinterpret_cast<int*>(base + w.vcnt);
  a.map_group = reinterpret_cast<int*>(base + w.share);
  a.vsel_stride = std::max(idx->v_cap_max, 1);
  a.lse = const_cast<float*>(lse);
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.dq_accumulate = dq_accumulate != 0;
  a.col_tiles = (idx->v_cap_max + 63) / 64;
  // Column units of about 48 query blocks.  Consecutive units of a column
  // tile differ in the query range and go round-robin to the 8 XCDs; with a
  // range count that is a multiple of 8 every XCD would always get the same
  // ranges, and the early ranges carry little work (few columns start that
  // early), which left one XCD with over twice the work of another.  An odd
  // count spreads every column tile's ranges over all XCDs.  A striped call
  // over one rank's key chunk holds about 1/W of each list's columns, so few
  // column tiles have work: there units of about 16 query blocks keep more
  // of them in flight (their partial dK, dV go out with fp32 atomics).
  a.qrange_len = (c.W > 1 && !c.k_all) ? 16 : 48;
  a.qranges = (c.nqb + a.qrange_len - 1) / a.qrange_len;
  while (a.qranges > 1 && a.qranges % 2 == 0) {
    ++a.qrange_len;
    a.qranges = (c.nqb + a.qrange_len - 1) / a.qrange_len;
  }
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipSuccess;
  float* l2 = reinterpret_cast<float*>(base + w.lse2);
  a.o = o;
  a.o_f32 = o_f32 != 0;
  if (c.bf16) {
    // The dQ kernel runs first and writes delta (when none is given) and
    // LSE * log2(e) of its rows for the dK/dV kernels.
    if (!delta) {
      float* dws = reinterpret_cast<float*>(base + w.delta);
      a.delta_out = dws;
      delta = dws;
    }
    a.lse2_out = l2;
  } else {
    if (!delta) {
      float* dws = reinterpret_cast<float*>(base + w.delta);
      e = vs::launch_delta(o, c.so, o_f32 != 0, c.bf16, dout, c.sdo, dws, c.batch, c.n_q, c.h_q, c.d, s);
      delta = dws;
    }
    if (e == hipSuccess) e = vs::launch_lse_log2(lse, l2, (size_t)c.batch * c.h_q * c.n_q, s);
  }
  a.delta = delta;
  a.lse2 = l2;
  if (e == hipSuccess) e = vs::launch_prep_vertical(a, c.n_lists(), idx->v_ptr, idx->v_idx, s);
  if (e == hipSuccess && idx->row_mask) {
    uint32_t* un = reinterpret_cast<uint32_t*>(base + w.rm_union);
    a.rm_union = un;
    e = vs::launch_moba_union(idx->row_mask, un, c.batch * c.h_q * c.nqb, s);
  }
  if (e == hipSuccess) e = vs::launch_bwd(a, c.bf16, c.d, s);
  return hip_status(e, what);
}
}  // namespace

extern "C" {

vs_status vs_sparse_attn_bwd(const vs_problem* p, const void* q, const void* k, const void* v,
                             const void* o, int32_t o_f32, const void* dout, const float* lse,
                             const float* delta, const vs_index* idx, float* dq,
                             int32_t dq_accumulate, float* dk, float* dv, void* ws,
                             size_t ws_bytes, vs_stream_t stream) {
  return attn_bwd("vs_sparse_attn_bwd", p, q, k, v, o, o_f32, dout, lse, delta, idx, dq, dq_accumulate, dk,
                  dv, ws, ws_bytes, false, stream);
}

vs_status vs_sparse_attn_bwd_noalloc(const vs_problem* p, const void* q, const void* k, const void* v,
                                     const void* o, int32_t o_f32, const void* dout, const float* lse,
                                     const float* delta, const vs_index* idx, float* dq,
                                     int32_t dq_accumulate, float* dk, float* dv, vs_stream_t stream) {
  return attn_bwd("vs_sparse_attn_bwd_noalloc", p, q, k, v, o, o_f32, dout, lse, delta, idx, dq,
                  dq_accumulate, dk, dv, nullptr, 0, true, stream);
}

vs_status lse_merge(int32_t batch, int32_t n, int32_t heads, int32_t head_dim, float* o_acc,
                    float* lse_acc, const float* o_part, const float* lse_part,
                    vs_stream_t stream) {
  if (!o_acc || !lse_acc || !o_part || !lse_part)
    return fail(VS_ERR_NULL, "lse_merge pointer is NULL");
  if (batch < 0 || n < 0 || heads < 0) return fail(VS_ERR_SHAPE, "negative size");
  if (head_dim < 4 || head_dim > 256 || (head_dim & (head_dim - 1)) != 0)
    return fail(VS_ERR_UNSUPPORTED, "head_dim %d unsupported (power of two, 4..256)", head_dim);
  return hip_status(vs::launch_lse_merge(batch, n, heads, head_dim, o_acc, lse_acc, o_part,
                                         lse_part, (hipStream_t)stream),
                    "lse_merge");
}

vs_status vs_trace_enable(int32_t on) {
  std::lock_guard<std::mutex> lk(g_tmu);
  g_trace = on != 0;
  return ok();
}

vs_status vs_trace_collect(char* buf, size_t len) {
  if (!buf || len == 0) return fail(VS_ERR_NULL, "trace buffer is NULL");
  std::vector<TraceRec> recs;
  {
    std::lock_guard<std::mutex> lk(g_tmu);
    recs.swap(g_pending);
  }
  std::map<std::string, std::pair<long, double>> agg;
  hipError_t err = hipSuccess;
  for (const TraceRec& r : recs) {
    float ms = 0.f;
    hipError_t e = hipEventSynchronize(r.stop);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.start, r.stop);
    if (e != hipSuccess) err = e;
    auto& a = agg[r.name];
    a.first += 1;
    a.second += ms;
  }
  {
    std::lock_guard<std::mutex> lk(g_tmu);
    for (const TraceRec& r : recs) {
      g_pool.push_back(r.start);
      g_pool.push_back(r.stop);
    }
  }
  std::string out;
  for (const auto& kv : agg) {
    char line[256];
    snprintf(line, sizeof line, "%s %ld %.6f\n", kv.first.c_str(), kv.second.first, kv.second.second);
    out += line;
  }
  std::snprintf(buf, len, "%s", out.c_str());
  if (err != hipSuccess) return fail(VS_ERR_HIP, "trace events: %s", hipGetErrorString(err));
  return ok();
}

}  // extern "C"
