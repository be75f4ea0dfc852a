"""GPU parity of the XAttention block estimator and of attention on a block
selection (the alternative estimator of the MTraining paper note, appendix,
baseline settings, item 2), through the C ABI, against the CPU oracle.

The estimator is checked in three layers: the device block scores against the
oracle's fp64 scores; the device's counts and bitmap against the integer
decision recomputed from the device's own scores (exact); and the selection
against the oracle's, where a difference is allowed only at a certified near
tie.  The attention calls take the oracle's selection, packed into the bitmap
layout on the host, so their parity does not depend on those near ties.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from vs_cases import (XA_SCORE_RTOL, check_close, check_xattn_row, log, np64, pack_block_selection,
                      xattn_count_int)

pytestmark = pytest.mark.gpu

vs = pytest.importorskip("dynamic_sparse_attention_amd")


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


XA_CASES = {
    # name: (make_problem kwargs, threshold)
    "w2-n4096-t0.9": (dict(wid=2, n=4096), 0.9),
    # 33 query blocks: the last one half full and a second bitmap word
    "w2-n4160-ragged-t0.5": (dict(wid=2, n=4160, h_q=4, h_kv=1), 0.5),
    "w2-n2048-d64-t1.0": (dict(wid=2, n=2048, h_q=4, h_kv=1, d=64), 1.0),
    "w2-n1024-t0": (dict(wid=2, n=1024, h_q=2, h_kv=1), 0.0),
    "w2-n8192-gqa8-t0.9": (dict(wid=2, n=8192, h_q=8, h_kv=1), 0.9),
}

def _oracle_case(prob, threshold):
    q, k = np64(prob.q[0]), np64(prob.k[0])
    return oracle.estimate_index_xattn(q, k, prob.cu_seqlens, 128, 16, threshold, return_scores=True)


def pack_selection(sel_by_head, nI, dev):
    return pack_block_selection(sel_by_head, nI).to(dev)


def block_index(mask, dev, h_q):
    zeros = torch.zeros(h_q + 1, dtype=torch.int32, device=dev)
    empty = torch.zeros(1, dtype=torch.int32, device=dev)
    return vs.VsIndexT(zeros, empty, zeros, empty, 0, 0, mask, 128)


@pytest.mark.parametrize("name", list(XA_CASES))
def test_xattn_estimator(name):
    dev = _dev()
    kw, thr = XA_CASES[name]
    kw = dict(kw)
    prob = workloads.make_problem(kw.pop("wid"), **kw)
    hq, n = prob.h_q, prob.n
    nI = -(-n // 128)
    log(f"case xattn {name}: n={n} hq={hq} hkv={prob.h_kv} d={prob.d} threshold={thr}")
    osel, osc, ocnt = _oracle_case(prob, thr)
    gq, gk = prob.q.to(dev), prob.k.to(dev)
    gidx, gcnt, gsc = vs.estimate_index_xattn(gq, gk, thr, return_scores=True)
    torch.cuda.synchronize()
    gsel = gidx.block_selection(n).numpy()          # [hq, nI, nI]
    gcnt = gcnt[0].cpu().numpy()
    gsc = gsc[0].cpu().numpy()
    assert gsel.shape == (hq, nI, nI)
    worst = 0.0
    flips = swaps = 0
    for h in range(hq):
        s_o = osc[(h, 0)]
        sel_o = osel[(h, 0)][2][1]
        for I in range(nI):
            e, f, w, ref = check_xattn_row((name, h, I), s_o[I, :I + 1], gsc[h, I, :I + 1], gsel[h, I],
                                           gcnt[h, I], int(ocnt[(h, 0)][I]), thr)
            worst, flips, swaps = max(worst, e), flips + f, swaps + w
            if not f and not w:
                assert np.array_equal(ref, np.nonzero(sel_o[I])[0]), (name, h, I)
    log(f"  xattn {name}: score err/(1+s) max {worst:.2e}; counts exact; "
        f"certified boundary flips={flips}, near-tie swaps={swaps}")


def _attn_case(name, prob, sel_by_head, dev):
    """Forward and backward on a block selection against the oracle."""
    hq, n = prob.h_q, prob.n
    nI = -(-n // 128)
    empty = np.zeros(0, np.int64)
    index = {(h, 0): (empty, empty, (128, sel_by_head[h])) for h in range(hq)}
    q, k, v, do = (np64(t[0]) for t in (prob.q, prob.k, prob.v, prob.do))
    pos = np.arange(n)
    if n <= 4096:
        O, L = oracle.attn_fwd_dense(q, k, v, pos, pos, prob.cu_seqlens, index)
    else:
        O, L = oracle.attn_fwd_support(q, k, v, pos, pos, prob.cu_seqlens, index)
    D = oracle.bwd_delta(O, do)
    if n <= 4096:
        dq, dk, dv = oracle.attn_bwd_dense(q, k, v, do, L, D, pos, pos, prob.cu_seqlens, index)
    else:
        dq, dk, dv = oracle.attn_bwd_support(q, k, v, do, L, D, pos, pos, prob.cu_seqlens, index)
    bq, bk, bv = oracle.bwd_rounding_bounds(q, k, v, do, O, L, pos, pos, prob.cu_seqlens, index)
    idx = block_index(pack_selection(sel_by_head, nI, dev), dev, hq)
    gq, gk, gv, gdo = (t.to(dev) for t in (prob.q, prob.k, prob.v, prob.do))
    o, lse = vs.sparse_attn_fwd(gq, gk, gv, idx)
    gdq, gdk, gdv = vs.sparse_attn_bwd(gq, gk, gv, o, gdo, lse, idx)
    torch.cuda.synchronize()
    errs = [check_close(f"{name} O", O, np64(o[0]), prob.dtype, "o"),
            check_close(f"{name} LSE", L, lse[0].cpu().numpy().astype(np.float64), prob.dtype),
            check_close(f"{name} dQ", dq, np64(gdq[0]), prob.dtype, "grad", bq),
            check_close(f"{name} dK", dk, np64(gdk[0]), prob.dtype, "grad", bk),
            check_close(f"{name} dV", dv, np64(gdv[0]), prob.dtype, "grad", bv)]
    errs = [e for e in errs if e]
    assert not errs, errs


BLOCK_ATTN_CASES = {
    # name: (make_problem kwargs, selection)
    # the oracle's XAttention selection at threshold 0.9
    "xattn-w2-n4096": (dict(wid=2, n=4096), "xattn"),
    # seeded random blocks: diagonal blocks missing on some rows, empty rows,
    # a half last query block and two bitmap words
    "random-n4160": (dict(wid=2, n=4160, h_q=4, h_kv=1), "random"),
    # every causal block, 16 Q heads on one KV head: equal to dense causal
    # attention, and early key blocks collect up to 16 x 64 dK/dV tiles
    "full-gqa16-n4096": (dict(wid=2, n=4096, h_q=16, h_kv=1), "full"),
    "empty-n1024": (dict(wid=2, n=1024, h_q=2, h_kv=1), "empty"),
    "xattn-d64-n2048": (dict(wid=2, n=2048, h_q=4, h_kv=1, d=64), "xattn"),
}


@pytest.mark.parametrize("name", list(BLOCK_ATTN_CASES))
def test_block_selection_attention(name):
    dev = _dev()
    kw, kind = BLOCK_ATTN_CASES[name]
    kw = dict(kw)
    prob = workloads.make_problem(kw.pop("wid"), **kw)
    hq, n = prob.h_q, prob.n
    nI = -(-n // 128)
    tril = np.tril(np.ones((nI, nI), bool))
    if kind == "xattn":
        osel = _oracle_case(prob, 0.9)[0]
        sels = [osel[(h, 0)][2][1] for h in range(hq)]
    elif kind == "random":
        rng = np.random.default_rng(77)
        sels = []
        for h in range(hq):
            s = (rng.random((nI, nI)) < 0.35) & tril
            s[rng.random(nI) < 0.2] = False  # empty query blocks
            s[np.arange(nI), np.arange(nI)] &= rng.random(nI) < 0.6
            sels.append(s)
    elif kind == "full":
        sels = [tril.copy() for _ in range(hq)]
    else:
        sels = [np.zeros((nI, nI), bool) for _ in range(hq)]
    log(f"case block attention {name}: n={n} hq={hq} hkv={prob.h_kv} d={prob.d} "
        f"blocks={int(sum(s.sum() for s in sels))}")
    _attn_case(name, prob, sels, dev)


def test_xattn_then_attention_batch2():
    """Batch 2 (two seeded rows): the device estimator's bitmap rows per
    (batch, head) equal the oracle's selection of each row away from near
    ties, and attention on the oracle's selection matches per row."""
    dev = _dev()
    p1 = workloads.make_problem(2, n=2048, h_q=4, h_kv=1, seed=11)
    p2 = workloads.make_problem(2, n=2048, h_q=4, h_kv=1, seed=12)
    q = torch.cat([p1.q, p2.q])
    k = torch.cat([p1.k, p2.k])
    gidx, gcnt, gsc = vs.estimate_index_xattn(q.to(dev), k.to(dev), 0.9, return_scores=True)
    torch.cuda.synchronize()
    nI = 16
    gsel = gidx.block_selection(2048).numpy().reshape(2, 4, nI, nI)
    for b, p in enumerate((p1, p2)):
        osel, osc, _ = _oracle_case(p, 0.9)
        for h in range(4):
            err = np.abs(gsc[b, h].cpu().numpy().astype(np.float64) - osc[(h, 0)])
            assert np.all(np.tril(err) <= XA_SCORE_RTOL * (1 + osc[(h, 0)])), (b, h)
            for I in range(nI):
                kk, order = xattn_count_int(gsc[b, h, I, :I + 1].cpu().numpy(), 0.9)
                want = np.zeros(nI, bool)
                want[np.asarray(order[:kk], np.int64)] = True
                assert np.array_equal(gsel[b, h, I], want), (b, h, I)
    # attention, batch 2, on the oracle's selections
    sels = [[_oracle_case(p, 0.9)[0][(h, 0)][2][1] for h in range(4)] for p in (p1, p2)]
    words = 1
    mask = torch.cat([pack_selection(s, nI, dev) for s in sels]).view(2 * 4 * nI, words)
    zeros = torch.zeros(2 * 4 + 1, dtype=torch.int32, device=dev)
    empty = torch.zeros(1, dtype=torch.int32, device=dev)
    idx = vs.VsIndexT(zeros, empty, zeros, empty, 0, 0, mask, 128)
    v = torch.cat([p1.v, p2.v]).to(dev)
    do = torch.cat([p1.do, p2.do]).to(dev)
    gq, gk = q.to(dev), k.to(dev)
    o, lse = vs.sparse_attn_fwd(gq, gk, v, idx)
    gdq, gdk, gdv = vs.sparse_attn_bwd(gq, gk, v, o, do, lse, idx)
    torch.cuda.synchronize()
    empty_np = np.zeros(0, np.int64)
    pos = np.arange(2048)
    errs = []
    for b, p in enumerate((p1, p2)):
        index = {(h, 0): (empty_np, empty_np, (128, sels[b][h])) for h in range(4)}
        qq, kk_, vv, dd = (np64(t[0]) for t in (p.q, p.k, p.v, p.do))
        O, L = oracle.attn_fwd_dense(qq, kk_, vv, pos, pos, p.cu_seqlens, index)
        D = oracle.bwd_delta(O, dd)
        dq, dk, dv = oracle.attn_bwd_dense(qq, kk_, vv, dd, L, D, pos, pos, p.cu_seqlens, index)
        bq, bk, bv = oracle.bwd_rounding_bounds(qq, kk_, vv, dd, O, L, pos, pos, p.cu_seqlens, index)
        errs += [check_close(f"b{b} O", O, np64(o[b]), "bf16", "o"),
                 check_close(f"b{b} LSE", L, lse[b].cpu().numpy().astype(np.float64), "bf16"),
                 check_close(f"b{b} dQ", dq, np64(gdq[b]), "bf16", "grad", bq),
                 check_close(f"b{b} dK", dk, np64(gdk[b]), "bf16", "grad", bk),
                 check_close(f"b{b} dV", dv, np64(gdv[b]), "bf16", "grad", bv)]
    errs = [e for e in errs if e]
    assert not errs, errs
