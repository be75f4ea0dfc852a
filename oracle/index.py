"""Oracle, part 1: the Vertical-Slash index (test infrastructure only).

Follows the MTraining paper note, Algorithm 1 ("dynamic sparse training
head"), and MTraining (arXiv 2510.18830) §4.1:

* an observation window of the last ``last_q`` queries is scored against all
  keys with a causal softmax (Algorithm 1, first step);
* vertical scores are column sums of the window probabilities, at token
  granularity; slash scores are the window probability mass on each
  block-diagonal of the 64x64 block grid (§4.1 (ii): verticals per token,
  slashes pooled over 64x64 blocks);
* ``argtopk`` keeps the k highest scores; ties go to the lowest index;
* ``sparseformat`` turns (vertical columns, slash block-diagonals) into the
  attention mask: causal, and the column is selected or the block-diagonal is.

Positions are global token positions inside one batch row.  A segment
[a, e) is one packed document; its block index of position p is
beta(p) = floor((p - a) / B).
"""
from __future__ import annotations

import numpy as np


def _ceil_div(a: int, b: int) -> int:
    return -(-int(a) // int(b))


def capacities(v_budget: int, s_budget: int, seg_len: int, n_total: int, block: int):
    """Number of verticals and slash block-diagonals kept for one segment.

    Budgets are tokens over the whole packed row; a segment of length L gets
    ceil(k * L / N) of each, the slash share is turned into ceil(share / B)
    block-diagonals, and both are clipped to the number of candidates (L
    columns, ceil(L / B) block-diagonals).  With one segment this is
    (min(k_v, N), min(ceil(k_s / B), N / B)).
    """
    share_v = _ceil_div(v_budget * seg_len, n_total)
    share_s = _ceil_div(s_budget * seg_len, n_total)
    nb = _ceil_div(seg_len, block)
    return min(share_v, seg_len), min(_ceil_div(share_s, block), nb)


def window_probs(q_h: np.ndarray, k_h: np.ndarray, a: int, e: int, scale: float, last_q: int):
    """Observation-window attention probabilities A_hat (Algorithm 1, first step).

    q_h: [N, d], k_h: [N, d] float64 rows of one head.  The window is the last
    w = min(last_q, L) rows of the segment [a, e).  Each window row r is a
    softmax over the keys a <= m <= r.  Returns (rows, A_hat [w, L], lse [w]).
    """
    w = min(last_q, e - a)
    rows = np.arange(e - w, e)
    cols = np.arange(a, e)
    s = scale * (q_h[rows] @ k_h[a:e].T)
    causal = cols[None, :] <= rows[:, None]
    s = np.where(causal, s, -np.inf)
    mx = s.max(axis=1)
    lse = mx + np.log(np.exp(s - mx[:, None]).sum(axis=1))
    probs = np.exp(s - lse[:, None])
    return rows, probs, lse


def window_scores(q_h, k_h, a, e, scale, block, last_q):
    """Vertical scores v[m] (token columns) and slash scores sigma[g] (block-diagonals).

    v[m] = sum over window rows of A_hat[r, m] (Algorithm 1, ``sum_v``).
    sigma[g] = sum of A_hat[r, m] over window entries whose block offset
    beta(r) - beta(m) equals g (``sum_s`` pooled on the 64x64 grid, §4.1 (ii)).
    Returns (v [L] indexed by m - a, sigma [nb]).
    """
    rows, probs, _ = window_probs(q_h, k_h, a, e, scale, last_q)
    L = e - a
    nb = _ceil_div(L, block)
    v = probs.sum(axis=0)
    g = ((rows - a) // block)[:, None] - (np.arange(L) // block)[None, :]
    keep = probs > 0
    sigma = np.bincount(g[keep], weights=probs[keep], minlength=nb)
    return v, sigma


def select_topk(scores: np.ndarray, k: int) -> np.ndarray:
    """``argtopk``: the k highest scores, ties to the lowest index, returned ascending."""
    k = min(int(k), scores.shape[0])
    order = np.lexsort((np.arange(scores.shape[0]), -scores))
    return np.sort(order[:k])


def topp_count(scores: np.ndarray, p: float) -> int:
    """``topp`` (Algorithm 1, budget lines): the fewest top scores that hold a
    fraction p of the total mass.

    With the scores sorted descending (ties to the lowest index, the order of
    ``argtopk``) and c their running sum, k = min{k : c[k-1] >= p * c[-1]};
    p <= 0 or an all-zero list gives 0.  c[-1] is the total, so p >= 1 gives
    the number of positive scores.  Reading of the pages (they define ``topp``
    only by name): the "minimal number of lines that recall a target
    proportion of the attention mass" of MTraining §4.1 (i).
    """
    s = np.asarray(scores, dtype=np.float64)
    if s.size == 0 or p <= 0:
        return 0
    order = np.lexsort((np.arange(s.size), -s))
    c = np.cumsum(s[order])
    total = c[-1]
    if total <= 0:
        return 0
    return int(np.argmax(c >= min(p, 1.0) * total)) + 1


def estimate_index_topp(q, k, cu_seqlens, v_cap, s_cap, p_v, p_s, block=64, last_q=64, scale=None,
                        return_scores=False):
    """Vertical-Slash index with top-p budgets (Algorithm 1: k_v = topp(sum_v, p_v),
    k_s = topp(pooled sum_s, p_s)), each capped by the fixed-budget capacity of
    ``capacities(v_cap[h], s_cap[h], ...)``.

    Returns {(h, seg): (iv, is_)} like ``estimate_index`` (lists of k_v <= cap
    and k_s <= cap entries) and, with return_scores, also the scores and the
    counts {(h, seg): (k_v, k_s)}.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    n, hq, d = q.shape
    hkv = k.shape[1]
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    out, scores, counts = {}, {}, {}
    for h in range(hq):
        g = h * hkv // hq
        for s in range(len(cu_seqlens) - 1):
            a, e = int(cu_seqlens[s]), int(cu_seqlens[s + 1])
            cv, cg = capacities(v_cap[h], s_cap[h], e - a, n, block)
            v, sigma = window_scores(q[:, h], k[:, g], a, e, scale, block, last_q)
            kv = min(topp_count(v, p_v[h]), cv)
            kg = min(topp_count(sigma, p_s[h]), cg)
            out[(h, s)] = (select_topk(v, kv) + a, select_topk(sigma, kg))
            scores[(h, s)] = (v, sigma)
            counts[(h, s)] = (kv, kg)
    return (out, scores, counts) if return_scores else out


def estimate_index(q, k, cu_seqlens, v_budget, s_budget, block=64, last_q=64, scale=None,
                   return_scores=False):
    """Vertical-Slash index for every (Q head, segment) of one batch row.

    q: [N, Hq, d], k: [N, Hkv, d] (any float dtype; computed in float64).
    Q head h reads KV head floor(h * Hkv / Hq) (grouped-query attention).
    v_budget / s_budget: per Q head, tokens.
    Returns {(h, seg): (iv, is_)} with iv global token positions (ascending)
    and is_ block-diagonal offsets g (ascending); optionally also the scores.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    n, hq, d = q.shape
    hkv = k.shape[1]
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    out, scores = {}, {}
    for h in range(hq):
        g = h * hkv // hq
        for s in range(len(cu_seqlens) - 1):
            a, e = int(cu_seqlens[s]), int(cu_seqlens[s + 1])
            kv, kg = capacities(v_budget[h], s_budget[h], e - a, n, block)
            v, sigma = window_scores(q[:, h], k[:, g], a, e, scale, block, last_q)
            out[(h, s)] = (select_topk(v, kv) + a, select_topk(sigma, kg))
            scores[(h, s)] = (v, sigma)
    return (out, scores) if return_scores else out


def _segment_of(pos, cu_seqlens):
    return np.searchsorted(np.asarray(cu_seqlens), pos, side="right") - 1


def block_selected(index_hs, n_off, m_off):
    """Entries whose (query block, key block) pair is selected in the optional
    block selection of an index entry (iv, is_, (bb, sel)): sel[I, J] marks key
    block J (of bb tokens, in-segment offsets m_off // bb) for query block I
    (n_off // bb).  An entry without that part selects no block."""
    n_off, m_off = np.asarray(n_off), np.asarray(m_off)
    if len(index_hs) < 3 or index_hs[2] is None:
        return np.zeros(np.broadcast(n_off, m_off).shape, dtype=bool)
    bb, sel = index_hs[2]
    sel = np.asarray(sel, dtype=bool)
    I, J = n_off // bb, m_off // bb
    ok = (I >= 0) & (J >= 0) & (I < sel.shape[0]) & (J < sel.shape[1])
    return ok & sel[np.clip(I, 0, sel.shape[0] - 1), np.clip(J, 0, sel.shape[1] - 1)]


def row_block_selected(index_hs, n_off, m_off):
    """Entries whose key block is picked for their row in the optional per-row
    block selection of an index entry (iv, is_, blk, (bb, sel)): sel[r, J]
    marks key block J (of bb tokens, in-segment offsets m_off // bb) for the
    row at in-segment offset r = n_off.  An entry without that part picks
    nothing."""
    n_off, m_off = np.broadcast_arrays(np.asarray(n_off), np.asarray(m_off))
    if len(index_hs) < 4 or index_hs[3] is None:
        return np.zeros(n_off.shape, dtype=bool)
    bb, sel = index_hs[3]
    sel = np.asarray(sel, dtype=bool)
    J = m_off // bb
    ok = (n_off >= 0) & (J >= 0) & (n_off < sel.shape[0]) & (J < sel.shape[1])
    return ok & sel[np.clip(n_off, 0, sel.shape[0] - 1), np.clip(J, 0, sel.shape[1] - 1)]


def dense_mask(rows_pos, cols_pos, cu_seqlens, index, h, block=64):
    """``sparseformat``: boolean mask [len(rows_pos), len(cols_pos)] for Q head h.

    M[n, m] holds when n and m lie in the same segment, m <= n (causal), and
    m is a selected vertical or beta(n) - beta(m) is a selected
    block-diagonal.  Vertical and slash entries form a union (Algorithm 1).
    An index entry may also carry a block selection (see block_selected) or
    a per-row block selection (see row_block_selected): their selected
    blocks join the union.
    rows_pos / cols_pos are global positions, so a striped chunk's mask is the
    global mask restricted to its rows and columns.
    """
    rows_pos = np.asarray(rows_pos)
    cols_pos = np.asarray(cols_pos)
    sr = _segment_of(rows_pos, cu_seqlens)
    sc = _segment_of(cols_pos, cu_seqlens)
    M = np.zeros((rows_pos.size, cols_pos.size), dtype=bool)
    for s in range(len(cu_seqlens) - 1):
        a = int(cu_seqlens[s])
        ri = np.nonzero(sr == s)[0]
        ci = np.nonzero(sc == s)[0]
        if ri.size == 0 or ci.size == 0:
            continue
        iv, is_ = index[(h, s)][:2]
        n = rows_pos[ri][:, None]
        m = cols_pos[ci][None, :]
        vert = np.isin(m, iv)
        slash = np.isin((n - a) // block - (m - a) // block, is_)
        blk = block_selected(index[(h, s)], n - a, m - a)
        rblk = row_block_selected(index[(h, s)], n - a, m - a)
        M[np.ix_(ri, ci)] = (m <= n) & (vert | slash | blk | rblk)
    return M
