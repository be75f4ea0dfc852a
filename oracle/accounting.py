"""Oracle, part 3: effective mask area (test infrastructure only).

Work is counted as the number of valid (row, column) entries of the mask, the
"effective mask area" of MagiAttention's "Dynamic Attention Solver" docs
("Computation Cost Estimation"): a full B x B block has B*B entries and a
causal diagonal block B(B+1)/2.
"""
from __future__ import annotations

import numpy as np

from .index import dense_mask


def mask_area_bruteforce(rows_pos, cols_pos, cu_seqlens, index, hq, block=64):
    """Count valid entries per Q head by building the dense mask."""
    return [int(dense_mask(rows_pos, cols_pos, cu_seqlens, index, h, block).sum())
            for h in range(hq)]


def mask_area_formula(cu_seqlens, index, hq, block=64):
    """Count valid entries per Q head from the index alone (contiguous layout).

    Per segment and query block i: every selected g <= i contributes the
    block pair (i, i-g): rows x columns, or the causal triangle when g = 0.
    Each selected vertical column m with beta(m) <= i whose block offset is
    not selected contributes the rows n >= m of block i.
    """
    out = []
    for h in range(hq):
        tot = 0
        for s in range(len(cu_seqlens) - 1):
            a, e = int(cu_seqlens[s]), int(cu_seqlens[s + 1])
            L = e - a
            nb = -(-L // block)
            iv, is_ = index[(h, s)]
            sel = set(int(g) for g in is_)
            bsize = [min(block, L - j * block) for j in range(nb)]
            for i in range(nb):
                ri = bsize[i]
                for g in sel:
                    if g > i:
                        continue
                    if g == 0:
                        tot += ri * (ri + 1) // 2
                    else:
                        tot += ri * bsize[i - g]
                r0 = a + i * block
                for m in iv:
                    bm = (int(m) - a) // block
                    if bm > i or (i - bm) in sel:
                        continue
                    # rows n in [r0, r0 + ri) with n >= m
                    tot += max(0, r0 + ri - max(int(m), r0))
        out.append(tot)
    return out


def dense_causal_area(rows_pos, cu_seqlens):
    """Causal area of the call's rows: each row n sees n - a + 1 keys of its segment."""
    rows_pos = np.asarray(rows_pos, dtype=np.int64)
    seg = np.searchsorted(np.asarray(cu_seqlens), rows_pos, side="right") - 1
    a = np.asarray(cu_seqlens, dtype=np.int64)[seg]
    return int((rows_pos - a + 1).sum())
