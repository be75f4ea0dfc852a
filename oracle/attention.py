"""Oracle, part 2: masked softmax attention, its backward, and the LSE merge.

Test infrastructure only.  Everything is float64.

Forward (MTraining arXiv 2510.18830 §3.2; Algorithm 1 last step): with
S = scale * Q K^T on the mask and -inf elsewhere, LSE[n] = log sum_m e^S[n,m]
(natural log; -inf for a row with no entry), A = e^(S - LSE), O = A V.

Backward (MTraining §3.2 Eq. 1-2; paper note Appendix B.1), with dO given:
dA = dO V^T, D = rowsum(dA * A) = rowsum(dO * O), dS = A * (dA - D),
dQ = scale dS K, dK = scale dS^T Q, dV = A^T dO.  A is rebuilt from the LSE
that the caller passes (the final, merged one when KV arrives in chunks — the
recompute-from-LSE scheme of "Ring Attention Paper Analysis", "Backward Pass
and Gradient Computation").  Grouped-query attention: Q head h uses KV head
floor(h * Hkv / Hq); dK and dV sum over the Q heads of a group.

Two evaluation forms compute the same numbers:
  (i)  ``*_dense``: the full [rows, cols] mask per head (small inputs);
  (ii) ``*_support``: per group of rows sharing a segment and a block, only
       the candidate keys of the Vertical-Slash index, with the mask
       definition evaluated on them; every other entry is exactly zero.
"""
from __future__ import annotations

import numpy as np

from .index import block_selected, dense_mask, row_block_selected, _segment_of


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def _softmax_rows(S):
    """Row-wise LSE of a score matrix with -inf holes (-inf for an empty row)."""
    if S.shape[1] == 0:
        return np.full(S.shape[0], -np.inf)
    mx = S.max(axis=1)
    empty = ~np.isfinite(mx)
    mx_safe = np.where(empty, 0.0, mx)
    Z = np.exp(S - mx_safe[:, None]).sum(axis=1)
    with np.errstate(divide="ignore"):
        lse = np.where(empty, -np.inf, mx_safe + np.log(np.where(empty, 1.0, Z)))
    return lse


def _probs(S, lse):
    lse_safe = np.where(np.isfinite(lse), lse, 0.0)
    P = np.exp(S - lse_safe[:, None])
    P[~np.isfinite(lse)] = 0.0
    return P


def attn_fwd_dense(q, k, v, rows_pos, cols_pos, cu_seqlens, index, block=64, scale=None):
    """Form (i) forward.  q [nr, Hq, d], k/v [nc, Hkv, d].  Returns O [nr, Hq, d], LSE [Hq, nr]."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    nr, hq, d = q.shape
    hkv = k.shape[1]
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    O = np.zeros((nr, hq, v.shape[2]))
    LSE = np.zeros((hq, nr))
    for h in range(hq):
        g = h * hkv // hq
        M = dense_mask(rows_pos, cols_pos, cu_seqlens, index, h, block)
        S = np.where(M, scale * (q[:, h] @ k[:, g].T), -np.inf)
        lse = _softmax_rows(S)
        A = _probs(S, lse)
        O[:, h] = A @ v[:, g]
        LSE[h] = lse
    return O, LSE


def attn_bwd_dense(q, k, v, do, lse, delta, rows_pos, cols_pos, cu_seqlens, index, block=64,
                   scale=None):
    """Form (i) backward.  lse / delta: [Hq, nr] (final values).  Returns dQ, dK, dV."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    lse, delta = _f64(lse), _f64(delta)
    nr, hq, d = q.shape
    hkv = k.shape[1]
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for h in range(hq):
        g = h * hkv // hq
        M = dense_mask(rows_pos, cols_pos, cu_seqlens, index, h, block)
        S = np.where(M, scale * (q[:, h] @ k[:, g].T), -np.inf)
        A = _probs(S, lse[h])
        dA = do[:, h] @ v[:, g].T
        dS = A * (dA - delta[h][:, None])
        dq[:, h] = scale * dS @ k[:, g]
        dk[:, g] += scale * dS.T @ q[:, h]
        dv[:, g] += A.T @ do[:, h]
    return dq, dk, dv


def row_groups(rows_pos, cu_seqlens, block=64):
    """Split the call's rows into groups that share a segment and a block index.

    Yields (row indices into rows_pos, segment, beta) with beta = floor((p - a)/B).
    """
    rows_pos = np.asarray(rows_pos)
    seg = _segment_of(rows_pos, cu_seqlens)
    a = np.asarray(cu_seqlens)[seg]
    beta = (rows_pos - a) // block
    key = seg.astype(np.int64) * (1 << 32) + beta
    order = np.argsort(key, kind="stable")
    bounds = np.nonzero(np.diff(key[order]))[0] + 1
    for grp in np.split(order, bounds):
        if grp.size:
            yield grp, int(seg[grp[0]]), int(beta[grp[0]])


def support_candidates(seg, beta, rows_max, cols_pos, cu_seqlens, index_hs, block=64):
    """Column indices (into cols_pos) that may hold an entry for rows of (seg, beta).

    The candidates are the key blocks beta - g for selected g, the selected
    vertical columns m <= rows_max, the keys of the blocks selected for the
    rows' block in the optional block selection, and the keys (<= rows_max)
    of the blocks any row of the block picked in the optional per-row block
    selection, restricted to the call's columns.  The caller evaluates the exact mask on them.
    """
    cols_pos = np.asarray(cols_pos)
    a, e = int(cu_seqlens[seg]), int(cu_seqlens[seg + 1])
    iv, is_ = index_hs[:2]
    want = []
    for g in is_:
        kb = beta - int(g)
        if kb < 0:
            continue
        lo = a + kb * block
        want.append(np.arange(lo, min(lo + block, e)))
    if len(index_hs) > 2 and index_hs[2] is not None:
        bb, sel = index_hs[2]
        I = (beta * block) // bb
        if I < len(sel):
            for J in np.nonzero(np.asarray(sel[I]))[0]:
                lo = a + int(J) * bb
                want.append(np.arange(lo, min(lo + bb, e)))
    if len(index_hs) > 3 and index_hs[3] is not None:
        bb, sel = index_hs[3]
        sel = np.asarray(sel, dtype=bool)
        rows = sel[beta * block:min((beta + 1) * block, sel.shape[0])]
        for J in np.nonzero(rows.any(axis=0))[0]:
            lo = a + int(J) * bb
            want.append(np.arange(lo, min(lo + bb, e, rows_max + 1)))
    want.append(np.asarray(iv)[np.asarray(iv) <= rows_max])
    want = np.unique(np.concatenate(want)) if want else np.zeros(0, np.int64)
    idx = np.searchsorted(cols_pos, want)
    idx = np.clip(idx, 0, max(cols_pos.size - 1, 0))
    ok = cols_pos.size > 0
    hit = (cols_pos[idx] == want) if ok else np.zeros(want.shape, bool)
    return idx[hit]


def _group_mask(rows_pos_g, cand_pos, seg, cu_seqlens, index_hs, block):
    a, e = int(cu_seqlens[seg]), int(cu_seqlens[seg + 1])
    iv, is_ = index_hs[:2]
    n = rows_pos_g[:, None]
    m = cand_pos[None, :]
    inseg = (m >= a) & (m < e)
    vert = np.isin(m, iv)
    slash = np.isin((n - a) // block - (m - a) // block, is_)
    blk = block_selected(index_hs, n - a, m - a)
    rblk = row_block_selected(index_hs, n - a, m - a)
    return inseg & (m <= n) & (vert | slash | blk | rblk)


def attn_fwd_support(q, k, v, rows_pos, cols_pos, cu_seqlens, index, block=64, scale=None,
                     heads=None, row_filter=None):
    """Form (ii) forward over the index's support only.

    cols_pos must be ascending.  ``heads`` limits the Q heads computed;
    ``row_filter(seg, beta)`` -> bool limits the row groups (sampling).
    Rows not computed are left NaN.  Returns O [nr, Hq, d], LSE [Hq, nr].
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    rows_pos = np.asarray(rows_pos)
    cols_pos = np.asarray(cols_pos)
    nr, hq, d = q.shape
    hkv = k.shape[1]
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    O = np.full((nr, hq, v.shape[2]), np.nan)
    LSE = np.full((hq, nr), np.nan)
    heads = range(hq) if heads is None else heads
    groups = list(row_groups(rows_pos, cu_seqlens, block))
    for h in heads:
        g = h * hkv // hq
        for ri, seg, beta in groups:
            if row_filter is not None and not row_filter(seg, beta):
                continue
            ci = support_candidates(seg, beta, rows_pos[ri].max(), cols_pos, cu_seqlens,
                                    index[(h, seg)], block)
            M = _group_mask(rows_pos[ri], cols_pos[ci], seg, cu_seqlens, index[(h, seg)], block)
            S = np.where(M, scale * (q[ri, h] @ k[ci, g].T), -np.inf)
            lse = _softmax_rows(S)
            A = _probs(S, lse)
            O[ri, h] = A @ v[ci, g]
            LSE[h, ri] = lse
    return O, LSE


def attn_bwd_support(q, k, v, do, lse, delta, rows_pos, cols_pos, cu_seqlens, index, block=64,
                     scale=None, heads=None, row_filter=None):
    """Form (ii) backward over the support.  Same contract as ``attn_bwd_dense``.

    ``row_filter(seg, beta)`` limits the row groups (sampling): dQ is then exact
    for the kept rows, and dK / dV hold only the kept rows' contributions.
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    lse, delta = _f64(lse), _f64(delta)
    rows_pos = np.asarray(rows_pos)
    cols_pos = np.asarray(cols_pos)
    nr, hq, d = q.shape
    hkv = k.shape[1]
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    heads = range(hq) if heads is None else heads
    groups = list(row_groups(rows_pos, cu_seqlens, block))
    for h in heads:
        g = h * hkv // hq
        for ri, seg, beta in groups:
            if row_filter is not None and not row_filter(seg, beta):
                continue
            ci = support_candidates(seg, beta, rows_pos[ri].max(), cols_pos, cu_seqlens,
                                    index[(h, seg)], block)
            if ci.size == 0:
                continue
            M = _group_mask(rows_pos[ri], cols_pos[ci], seg, cu_seqlens, index[(h, seg)], block)
            S = np.where(M, scale * (q[ri, h] @ k[ci, g].T), -np.inf)
            A = _probs(S, lse[h, ri])
            dA = do[ri, h] @ v[ci, g].T
            dS = A * (dA - delta[h, ri][:, None])
            dq[ri, h] = scale * dS @ k[ci, g]
            dk[ci, g] += scale * dS.T @ q[ri, h]
            dv[ci, g] += A.T @ do[ri, h]
    return dq, dk, dv


def lse_merge(o1, lse1, o2, lse2):
    """``merge_out_and_lse`` (paper note Appendix E, Algorithm 2).

    For each row: LSE = max + log(e^(l1 - max) + e^(l2 - max)) and
    O = e^(l1 - LSE) O1 + e^(l2 - LSE) O2, the exact combination of two
    softmax-normalised partial results over disjoint key sets.  A partial
    with LSE = -inf (no keys) is the identity; two of them give (O = 0,
    LSE = -inf).  o*: [..., rows, d] with lse*: [..., rows].
    """
    o1, o2, lse1, lse2 = _f64(o1), _f64(o2), _f64(lse1), _f64(lse2)
    mx = np.maximum(lse1, lse2)
    both_empty = ~np.isfinite(mx)
    mx_safe = np.where(both_empty, 0.0, mx)
    w1 = np.where(np.isfinite(lse1), np.exp(lse1 - mx_safe), 0.0)
    w2 = np.where(np.isfinite(lse2), np.exp(lse2 - mx_safe), 0.0)
    tot = w1 + w2
    with np.errstate(divide="ignore"):
        lse = np.where(both_empty, -np.inf, mx_safe + np.log(np.where(both_empty, 1.0, tot)))
    tot_safe = np.where(both_empty, 1.0, tot)
    o = (w1 / tot_safe)[..., None] * o1 + (w2 / tot_safe)[..., None] * o2
    return o, lse


def bwd_delta(o, do):
    """D[h, n] = rowsum(dO * O), which equals rowsum(dA * A) of Eq. 1 (MTraining §3.2).

    o, do: [rows, Hq, d].  Returns [Hq, rows] float64.
    """
    return (_f64(o) * _f64(do)).sum(-1).T


def bwd_rounding_bounds(q, k, v, do, o, lse, rows_pos, cols_pos, cu_seqlens, index, block=64,
                        scale=None, u_op=2.0 ** -8, u_o=2.0 ** -8, support=None, row_filter=None):
    """First-order error bounds of a backward whose matrix-core operands P and dS
    are rounded to a format of unit roundoff u_op, with delta formed from an
    output O that was itself computed with P rounded to u_op (O = P V) and
    stored with unit roundoff u_o (bf16: 2^-8 each; MTraining §5.1 trains in
    bfloat16).  Inputs are taken as exact.

    With |e_O| <= u_o |O| + u_op P |V| and D~ = D + e_D,
    |e_D| <= sum_c |dO| e_O, and dS~ = P (dP - D~) rounded:
      |dQ~ - dQ| <= scale * (u_op |dS| |K| + |e_D| P |K|)
      |dK~ - dK| <= scale * (u_op |dS|^T |Q| + (P |e_D|)^T |Q|)
      |dV~ - dV| <= u_op P^T |dO|
    (row-wise sums over the support; GQA sums over the group).  Returns
    (bq, bk, bv) shaped like dQ, dK, dV.  ``support`` selects form (ii) when
    True (default: form (i) for at most 4096 rows).  ``row_filter(seg, beta)``
    (form (ii) only) keeps the row groups it accepts, as in ``attn_bwd_support``.
    """
    q, k, v, do, o = _f64(q), _f64(k), _f64(v), _f64(do), _f64(o)
    lse = _f64(lse)
    rows_pos = np.asarray(rows_pos)
    cols_pos = np.asarray(cols_pos)
    nr, hq, d = q.shape
    hkv = k.shape[1]
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    use_support = (nr > 4096) if support is None else support
    if row_filter is not None:
        use_support = True
    D = bwd_delta(o, do)
    bq = np.zeros_like(q)
    bk = np.zeros_like(k)
    bv = np.zeros_like(v)
    aq, ak, av, ado, ao = np.abs(q), np.abs(k), np.abs(v), np.abs(do), np.abs(o)

    def accumulate(h, g, ri, ci, M):
        S = np.where(M, scale * (q[ri, h] @ k[ci, g].T), -np.inf)
        A = _probs(S, lse[h, ri])
        dA = do[ri, h] @ v[ci, g].T
        adS = np.abs(A * (dA - D[h, ri][:, None]))
        eO = u_o * ao[ri, h] + u_op * (A @ av[ci, g])
        e = (ado[ri, h] * eO).sum(-1)
        bq[ri, h] = scale * (u_op * adS @ ak[ci, g] + e[:, None] * (A @ ak[ci, g]))
        bk[ci, g] += scale * (u_op * adS.T @ aq[ri, h] + (A * e[:, None]).T @ aq[ri, h])
        bv[ci, g] += u_op * A.T @ ado[ri, h]

    for h in range(hq):
        g = h * hkv // hq
        if not use_support:
            M = dense_mask(rows_pos, cols_pos, cu_seqlens, index, h, block)
            accumulate(h, g, np.arange(nr), np.arange(cols_pos.size), M)
            continue
        for ri, seg, beta in row_groups(rows_pos, cu_seqlens, block):
            if row_filter is not None and not row_filter(seg, beta):
                continue
            ci = support_candidates(seg, beta, rows_pos[ri].max(), cols_pos, cu_seqlens,
                                    index[(h, seg)], block)
            if ci.size == 0:
                continue
            M = _group_mask(rows_pos[ri], cols_pos[ci], seg, cu_seqlens, index[(h, seg)], block)
            accumulate(h, g, ri, ci, M)
    return bq, bk, bv
