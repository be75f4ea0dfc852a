"""Work accounting of a Vertical-Slash index (host side, numpy).

The work of sparse attention is the number of valid (row, key) entries, the
"effective mask area" of the MagiAttention "Dynamic Attention Solver" docs
("Computation Cost Estimation"): each selected block-diagonal g > 0 adds one
full 64x64 block per query block i >= g, g = 0 adds the causal triangle
64*65/2 per block, and each selected column m adds, for every query block at
or below it whose offset to m's block is not selected, its rows n >= m.

FLOP conventions: forward 4*d per entry (two products), backward 10*d per
entry (five products: S recompute, dP, dV, dQ, dK).
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

FWD_FLOPS_PER_ENTRY_PER_DIM = 4
BWD_FLOPS_PER_ENTRY_PER_DIM = 10


def executed_split(lists, cu_seqlens: Sequence[int], h_q: int, block: int = 64,
                   row_blocks: Optional[np.ndarray] = None):
    """Valid entries per Q head, split into slash-block entries and vertical-column
    entries (columns inside a selected block count once, as slash entries).

    lists[l] = (verticals, block-diagonals), l = h * n_seg + s (batch 1).
    row_blocks: optional global block indices of the rows actually held
    (one segment only, e.g. a block-striped worker); default all rows.
    Returns {"slash": int64[h_q], "vertical": int64[h_q]}.
    """
    n_seg = len(cu_seqlens) - 1
    sl = np.zeros(h_q, dtype=np.int64)
    ve = np.zeros(h_q, dtype=np.int64)
    tri = block * (block + 1) // 2
    for h in range(h_q):
        for s in range(n_seg):
            a, e = int(cu_seqlens[s]), int(cu_seqlens[s + 1])
            nb = (e - a) // block
            iv, is_ = lists[h * n_seg + s]
            iv = np.asarray(iv, dtype=np.int64)
            iv = iv[iv >= 0]
            is_ = np.asarray(is_, dtype=np.int64)
            is_ = np.sort(is_[(is_ >= 0) & (is_ < nb)])
            rows = np.arange(nb, dtype=np.int64) if row_blocks is None else \
                np.asarray(row_blocks, dtype=np.int64)
            # slash part: blocks (i, i - g) for g <= i
            cnt_le = np.searchsorted(is_, rows, side="right")      # #g <= i
            has0 = is_.size > 0 and is_[0] == 0
            sl[h] += int((cnt_le - (1 if has0 else 0)).clip(min=0).sum()) * block * block
            if has0:
                sl[h] += rows.size * tri
            if iv.size == 0:
                continue
            bm = (iv - a) // block
            if row_blocks is None:
                # rows of m's own block at or below m, unless offset 0 is selected
                if not has0:
                    ve[h] += int((a + (bm + 1) * block - iv).sum())
                # later blocks: offsets 1 .. nb-1-bm not selected
                span = nb - 1 - bm
                nsel = np.searchsorted(is_, span, side="right") - np.searchsorted(is_, 1, side="left")
                ve[h] += int(((span - nsel).clip(min=0)).sum()) * block
            else:
                selset = np.zeros(nb + 1, dtype=bool)
                selset[is_] = True
                for i in rows:
                    off = i - bm
                    ok = (off >= 0) & ~selset[np.clip(off, 0, nb)]
                    full = ok & (off > 0)
                    same = ok & (off == 0)
                    ve[h] += int(full.sum()) * block
                    ve[h] += int((a + (i + 1) * block - iv[same]).sum())
    return {"slash": sl, "vertical": ve}


def executed_area(lists, cu_seqlens: Sequence[int], h_q: int, block: int = 64,
                  row_blocks: Optional[np.ndarray] = None) -> np.ndarray:
    """Valid entries per Q head (slash and vertical entries together)."""
    sp = executed_split(lists, cu_seqlens, h_q, block, row_blocks)
    return sp["slash"] + sp["vertical"]


def dense_causal_area(cu_seqlens: Sequence[int], row_positions: Optional[np.ndarray] = None) -> int:
    """Causal entries per head: sum over rows of (position - segment start + 1)."""
    if row_positions is None:
        return int(sum((e - a) * (e - a + 1) // 2 for a, e in zip(cu_seqlens[:-1], cu_seqlens[1:])))
    rp = np.asarray(row_positions, dtype=np.int64)
    seg = np.searchsorted(np.asarray(cu_seqlens), rp, side="right") - 1
    return int((rp - np.asarray(cu_seqlens, dtype=np.int64)[seg] + 1).sum())


def block_selection_area(sel: np.ndarray, n: int, blk: int = 128) -> np.ndarray:
    """Valid entries per row of a block selection sel [..., nI, nI] (bool) of
    one n-token segment: a selected block J < I adds rows(I) x blk entries, a
    selected diagonal block its causal triangle rows(I) (rows(I) + 1) / 2,
    rows(I) = min(blk, n - blk I).  Returns int64 [...] (e.g. per head)."""
    sel = np.asarray(sel, dtype=bool)
    nI = sel.shape[-1]
    rows = np.minimum(blk, n - blk * np.arange(nI, dtype=np.int64))
    below = np.tril(np.ones((nI, nI), dtype=bool), -1)
    off = (sel & below).sum(axis=-1).astype(np.int64)           # [..., nI] blocks J < I
    diag = np.diagonal(sel, axis1=-2, axis2=-1).astype(np.int64)
    return (off * rows * blk + diag * rows * (rows + 1) // 2).sum(axis=-1)


def row_selection_area(words: np.ndarray, n: int, blk: int) -> np.ndarray:
    """Valid entries per leading index of per-row block selections
    words [..., n] (bit J of a row's word picks key block J of blk tokens):
    row r counts, for each picked block J, its keys m <= r.  Returns int64 [...]."""
    w = np.asarray(words).astype(np.int64) & 0xFFFFFFFF
    lead = w.shape[:-1]
    w = w.reshape(-1, n)
    nB = -(-n // blk)
    r = np.arange(n, dtype=np.int64)[:, None]
    J = np.arange(nB, dtype=np.int64)[None, :]
    keys = np.clip(np.minimum(r + 1, (J + 1) * blk) - J * blk, 0, None)   # [n, nB]
    out = np.empty(w.shape[0], dtype=np.int64)
    for i in range(w.shape[0]):
        bits = (w[i][:, None] >> J) & 1
        out[i] = int((bits * keys).sum())
    return out.reshape(lead)
