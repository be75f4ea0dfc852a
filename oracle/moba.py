"""Oracle, part 5: the MoBA block gate (test infrastructure only).

The MTraining paper note (appendix, baseline settings, item 1) describes the
MoBA baseline: the key sequence is cut into fixed-size blocks, an MoE-style
gate picks for every query the top-k most relevant blocks, always including
the query's own block, and attention runs inside the picked blocks; block
size 4096, top-k 12.  The note does not define the gate's score; the plainest
readings taken here:

  M1  Blocks: key block b of a segment [a, e) holds the keys a + B b ..
      a + B (b + 1) - 1 (B = 4096; the segment's last block may be short).
  M2  Gate score of block b for query row n: q_n . kbar_b, kbar_b the mean of
      the block's keys -- the block's single representative in the gate, as
      an expert's key in an MoE router.  A scale or a softmax over the blocks
      would not change the ranking, so none is applied.
  M3  Candidates: the blocks wholly before the query's own block (the gate
      never looks ahead); the own block is always picked.
  M4  Selection: the own block and the k - 1 highest-scoring earlier blocks
      (ties to the lowest index), or every earlier block when there are at
      most k - 1 of them.
  M5  Mask: row n attends key m iff both lie in the segment, m <= n, and m's
      block is picked for n; per Q head, K read through the GQA map.
"""
from __future__ import annotations

import numpy as np


def block_means(k_h, a, e, B):
    """kbar [nB, d]: the mean of each key block of segment [a, e) (M1, M2)."""
    L = e - a
    nB = -(-L // B)
    return np.stack([k_h[a + b * B:min(a + (b + 1) * B, e)].mean(axis=0) for b in range(nB)])


def gate_scores(q_h, k_h, a, e, B):
    """s [L, nB]: q_n . kbar_b for every row n of the segment and every block
    (M2); the selection only reads the blocks before the row's own."""
    return np.asarray(q_h[a:e], np.float64) @ block_means(np.asarray(k_h, np.float64), a, e, B).T


def select_blocks(s, B, topk):
    """sel [L, nB] bool (M3, M4): row r keeps its own block r // B and the
    topk - 1 highest-scoring blocks before it, ties to the lowest index."""
    L, nB = s.shape
    sel = np.zeros((L, nB), dtype=bool)
    for r in range(L):
        own = r // B
        sel[r, own] = True
        past = s[r, :own]
        order = np.lexsort((np.arange(own), -past))
        sel[r, order[:max(topk - 1, 0)]] = True
    return sel


def estimate_index_moba(q, k, cu_seqlens, block=4096, topk=12, return_scores=False):
    """MoBA block selection for every (Q head, segment) of one batch row.

    q: [N, Hq, d], k: [N, Hkv, d]; Q head h reads KV head h * Hkv // Hq.
    Returns {(h, seg): (no verticals, no block-diagonals, no block selection,
    (block, sel))} with sel [L, nB] the picked blocks of every row of the
    segment -- the per-row form the attention functions take -- and with
    return_scores also the gate scores {(h, seg): s [L, nB]}.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    n, hq, d = q.shape
    hkv = k.shape[1]
    empty = np.zeros(0, np.int64)
    out, scores = {}, {}
    for h in range(hq):
        g = h * hkv // hq
        for sg in range(len(cu_seqlens) - 1):
            a, e = int(cu_seqlens[sg]), int(cu_seqlens[sg + 1])
            s = gate_scores(q[:, h], k[:, g], a, e, block)
            out[(h, sg)] = (empty, empty, None, (block, select_blocks(s, block, topk)))
            scores[(h, sg)] = s
    return (out, scores) if return_scores else out
