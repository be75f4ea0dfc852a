"""Oracle, part 4: the XAttention block estimator (test infrastructure only).

The MTraining paper note (appendix, baseline settings, item 2) describes the
XAttention baseline as scoring square blocks of the attention matrix by sums
taken along their anti-diagonals at a stride, keeping only high-scoring
blocks, with block size 128, stride 16 and threshold 0.9.  The note leaves
the steps between those words open; the plainest readings taken here:

  X1  Sampling.  A block of B x B (B = 128) is covered by (B/S)^2 cells of
      S x S (S = 16).  The cell (A, C) of a segment [a, e) holds rows
      a + S A + i and keys a + S C + j, and is sampled along its
      anti-diagonal i + j = S - 1: pairs (a + S A + u, a + S C + S - 1 - u).
  X2  Cell logit.  z[A, C] = the mean of the sampled scaled scores,
      (1/S) sum_u scale * q . k (scale = 1/sqrt(d)), so that a cell logit is
      on the scale of one attention logit.
  X3  Causality at cell level: cell (A, C) takes part iff C <= A (the cell on
      the diagonal, whose anti-diagonal straddles it, included whole).
  X4  Normalisation: p[A, .] = softmax of z[A, .] over the cells C <= A of
      the cell row, as attention normalises a row over its causal keys.
  X5  Block score: s[I, J] = sum of p over the cells of block (I, J) (rows A
      with A // (B/S) = I, keys C with C // (B/S) = J).  Each cell row sums to
      1, so sum_J s[I, J] is the number of cell rows of block I.
  X6  Selection ("threshold 0.9 for selecting blocks"): for each query block
      I, the fewest key blocks J <= I whose scores, highest first (ties to the
      lowest J), sum to at least the threshold times sum_J s[I, J] -- the
      top-p rule of the Vertical-Slash budgets (``topp_count``) on block
      scores.
  X7  Mask: row n attends key m iff they share a segment, m <= n, and the
      block of m is selected for the block of n; per Q head and segment, as
      the Vertical-Slash index.
"""
from __future__ import annotations

import numpy as np

from .index import topp_count


def antidiag_logits(q_h, k_h, a, e, scale, stride):
    """Cell logits z [nC, nC] of segment [a, e) (X1, X2), nC = (e - a) / stride.

    q_h, k_h: [N, d] float64 rows of one head.  Entries above the cell
    diagonal are -inf (X3)."""
    L = e - a
    S = int(stride)
    if L % S:
        raise ValueError("segment length must be a multiple of the stride")
    nC = L // S
    qs = q_h[a:e].reshape(nC, S, -1)             # qs[A, u] = q[a + S A + u]
    ks = k_h[a:e].reshape(nC, S, -1)[:, ::-1]    # ks[C, u] = k[a + S C + S - 1 - u]
    z = np.zeros((nC, nC))
    for u in range(S):
        z += qs[:, u] @ ks[:, u].T
    z *= scale / S
    causal = np.arange(nC)[None, :] <= np.arange(nC)[:, None]
    return np.where(causal, z, -np.inf)


def xattn_block_scores(q_h, k_h, a, e, scale, stride=16, block=128):
    """Block scores s [nI, nI] of segment [a, e) (X4, X5); s[I, J] = 0 for J > I."""
    z = antidiag_logits(q_h, k_h, a, e, scale, stride)
    mx = z.max(axis=1, keepdims=True)
    p = np.exp(z - mx)
    p /= p.sum(axis=1, keepdims=True)
    nC = z.shape[0]
    cpb = block // stride                         # cells per block side
    nI = -(-nC // cpb)
    # s[I, J] = sum of p over the cells of block (I, J): pad the cell grid to
    # whole blocks with zero probability and sum each cpb x cpb tile
    padded = np.zeros((nI * cpb, nI * cpb))
    padded[:nC, :nC] = p
    s = padded.reshape(nI, cpb, nI, cpb).sum(axis=(1, 3))
    return np.tril(s)


def estimate_index_xattn(q, k, cu_seqlens, block=128, stride=16, threshold=0.9, scale=None,
                         return_scores=False):
    """XAttention block selection for every (Q head, segment) of one batch row.

    q: [N, Hq, d], k: [N, Hkv, d]; Q head h reads KV head h * Hkv // Hq.
    Returns {(h, seg): (no verticals, no block-diagonals, (block, sel))} with
    sel[I, J] the selected key blocks of query block I (X6), the form the
    attention functions take, and with return_scores also the block scores
    {(h, seg): s} and the counts {(h, seg): k per query block}.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    n, hq, d = q.shape
    hkv = k.shape[1]
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    empty = np.zeros(0, np.int64)
    out, scores, counts = {}, {}, {}
    for h in range(hq):
        g = h * hkv // hq
        for sg in range(len(cu_seqlens) - 1):
            a, e = int(cu_seqlens[sg]), int(cu_seqlens[sg + 1])
            s = xattn_block_scores(q[:, h], k[:, g], a, e, scale, stride, block)
            nI = s.shape[0]
            sel = np.zeros((nI, nI), dtype=bool)
            cnt = np.zeros(nI, np.int64)
            for I in range(nI):
                row = s[I, :I + 1]
                kk = topp_count(row, threshold)
                order = np.lexsort((np.arange(row.size), -row))
                sel[I, order[:kk]] = True
                cnt[I] = kk
            out[(h, sg)] = (empty, empty, (block, sel))
            scores[(h, sg)] = s
            counts[(h, sg)] = cnt
    return (out, scores, counts) if return_scores else out
