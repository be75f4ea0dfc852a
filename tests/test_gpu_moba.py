"""GPU parity of the MoBA block gate and of attention on a per-row block
selection (the paper note's appendix, baseline settings, item 1), through the
C ABI, against the CPU oracle.

The gate is checked in three layers: the device's gate scores against the
oracle's fp64 scores; the device's per-row words against the selection
recomputed from the device's own fp32 scores (exact); and the selection
against the oracle's, a difference allowed only where the oracle's scores of
the blocks that differ tie with the last picked one within the score bound.
The attention calls take the oracle's selection (or seeded host selections),
packed into row words on the host.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from vs_cases import check_close, log, np64

pytestmark = pytest.mark.gpu

vs = pytest.importorskip("dynamic_sparse_attention_amd")


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


# The device forms kbar in fp32 from up to `block` bf16 keys and the score as
# an fp32 sum of d products: its error is a small multiple of 2^-24 times
# sum_c |q_c| |kbar_c| (and of the summed keys' magnitude); the bar is
# 2^-12 of that sum.
SCORE_REL = 2.0 ** -12


def device_pick(scores_f32, own, topk):
    """The per-row word in the device's arithmetic from its fp32 scores: the
    own block and the topk - 1 best earlier blocks, ties to the lowest."""
    s = np.asarray(scores_f32, np.float32)[:own]
    order = np.lexsort((np.arange(own), -s.astype(np.float64)))
    word = 1 << own
    for J in order[:max(topk - 1, 0)]:
        word |= 1 << int(J)
    return word


def words_of(sel):
    """Row words of a selection sel [L, nB] (bool)."""
    sel = np.asarray(sel, bool)
    return (sel * (1 << np.arange(sel.shape[1], dtype=np.int64))[None, :]).sum(axis=1).astype(np.int64)


def check_gate(tag, q64, kh64, n, block, topk, s_dev, w_dev, osel, ostat):
    """One (batch, head): scores, exact words, selection vs the oracle."""
    kbar = oracle.block_means(kh64, 0, n, block)
    mag = np.abs(q64) @ np.abs(kbar).T
    s_o = ostat
    nB = kbar.shape[0]
    flips = 0
    worst = 0.0
    for r in range(n):
        own = r // block
        if own:
            err = np.abs(s_dev[r, :own].astype(np.float64) - s_o[r, :own])
            bound = SCORE_REL * mag[r, :own] + 1e-30
            worst = max(worst, float((err / bound).max()))
            assert np.all(err <= bound), (tag, r, float(err.max()))
        assert int(w_dev[r]) & 0xFFFFFFFF == device_pick(s_dev[r], own, topk), (tag, r)
        want = int(words_of(osel[r:r + 1])[0])
        got = int(w_dev[r]) & 0xFFFFFFFF
        if got != want:
            diff = [J for J in range(nB) if ((got ^ want) >> J) & 1]
            picked = [J for J in range(own) if (want >> J) & 1]
            kth = min(s_o[r, J] for J in picked) if picked else 0.0
            tol = 2 * SCORE_REL * (mag[r, :own].max() if own else 0.0)
            assert all(abs(s_o[r, J] - kth) <= tol for J in diff), (tag, r, "non-tie mismatch")
            flips += 1
    return worst, flips


GATE_CASES = {
    # name: (make_problem kwargs, block, topk)
    "w2-n4096-b256-k4": (dict(wid=2, n=4096), 256, 4),
    # 9 blocks, the last one 64 keys long
    "w2-n4160-b512-k3": (dict(wid=2, n=4160, h_q=4, h_kv=1), 512, 3),
    "w2-n2048-d64-b256-k2": (dict(wid=2, n=2048, h_q=4, h_kv=1, d=64), 256, 2),
    "w2-n2048-b256-k1": (dict(wid=2, n=2048, h_q=2, h_kv=1), 256, 1),
    "w2-n2048-b256-k8": (dict(wid=2, n=2048, h_q=2, h_kv=1), 256, 8),
}


@pytest.mark.parametrize("name", list(GATE_CASES))
def test_moba_gate(name):
    dev = _dev()
    kw, block, topk = GATE_CASES[name]
    kw = dict(kw)
    prob = workloads.make_problem(kw.pop("wid"), **kw)
    n, hq, hkv = prob.n, prob.h_q, prob.h_kv
    log(f"case moba gate {name}: n={n} hq={hq} hkv={hkv} d={prob.d} block={block} topk={topk}")
    q64, k64 = np64(prob.q[0]), np64(prob.k[0])
    osel, osc = oracle.estimate_index_moba(q64, k64, prob.cu_seqlens, block, topk, return_scores=True)
    gidx, gsc = vs.estimate_index_moba(prob.q.to(dev), prob.k.to(dev), block, topk, return_scores=True)
    torch.cuda.synchronize()
    words = gidx.row_mask[0].cpu().numpy()
    gsc = gsc[0].cpu().numpy()
    worst, flips = 0.0, 0
    for h in range(hq):
        g = h * hkv // hq
        w_, f_ = check_gate((name, h), q64[:, h], k64[:, g], n, block, topk, gsc[h], words[h],
                            osel[(h, 0)][3][1], osc[(h, 0)])
        worst, flips = max(worst, w_), flips + f_
    log(f"  moba {name}: score err/bound max {worst:.2e}; words exact; certified near-tie rows {flips}")


def row_index(words, block, dev, hq):
    """VsIndexT of per-row words [Hq, n] (batch 1)."""
    zeros = torch.zeros(hq + 1, dtype=torch.int32, device=dev)
    empty = torch.zeros(1, dtype=torch.int32, device=dev)
    w = torch.from_numpy(np.asarray(words, np.int64).astype(np.uint32).view(np.int32)).to(dev)
    return vs.VsIndexT(zeros, empty, zeros, empty, 0, 0, row_mask=w.reshape(1, hq, -1).contiguous(),
                       row_blk=block)


def _attn_case(name, prob, sels, block, dev, batch_rows=None):
    hq, n = prob.h_q, prob.n
    empty = np.zeros(0, np.int64)
    index = {(h, 0): (empty, empty, None, (block, sels[h])) for h in range(hq)}
    q, k, v, do = (np64(t[0]) for t in (prob.q, prob.k, prob.v, prob.do))
    pos = np.arange(n)
    O, L = oracle.attn_fwd_dense(q, k, v, pos, pos, prob.cu_seqlens, index)
    D = oracle.bwd_delta(O, do)
    dq, dk, dv = oracle.attn_bwd_dense(q, k, v, do, L, D, pos, pos, prob.cu_seqlens, index)
    bq, bk, bv = oracle.bwd_rounding_bounds(q, k, v, do, O, L, pos, pos, prob.cu_seqlens, index)
    idx = row_index(np.stack([words_of(s) for s in sels]), block, dev, hq)
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


ROW_CASES = {
    # name: (make_problem kwargs, block, selection)
    "gate-w2-n4096-b256-k4": (dict(wid=2, n=4096), 256, ("gate", 4)),
    "gate-n4160-b512-k3": (dict(wid=2, n=4160, h_q=4, h_kv=1), 512, ("gate", 3)),
    "gate-d64-n2048-b256-k2": (dict(wid=2, n=2048, h_q=4, h_kv=1, d=64), 256, ("gate", 2)),
    # seeded selections: rows without their own block, rows picking nothing
    # (empty rows), 16 Q heads on one KV head so the dK/dV tile list flushes
    "random-gqa16-n4096-b256": (dict(wid=2, n=4096, h_q=16, h_kv=1), 256, ("random", None)),
    "own-only-n2048-b256": (dict(wid=2, n=2048, h_q=2, h_kv=1), 256, ("gate", 1)),
    # 64-token row blocks: the two key blocks of a dK/dV pair carry different
    # picks; 128-token row blocks with an odd key-block count (63)
    "random-n2048-b64": (dict(wid=2, n=2048, h_q=4, h_kv=1), 64, ("random", None)),
    "random-n4032-b128-odd": (dict(wid=2, n=4032, h_q=4, h_kv=2), 128, ("random", None)),
}


@pytest.mark.parametrize("name", list(ROW_CASES))
def test_row_selection_attention(name):
    dev = _dev()
    kw, block, (kind, topk) = ROW_CASES[name]
    kw = dict(kw)
    prob = workloads.make_problem(kw.pop("wid"), **kw)
    n, hq = prob.n, prob.h_q
    nB = -(-n // block)
    if kind == "gate":
        osel = oracle.estimate_index_moba(np64(prob.q[0]), np64(prob.k[0]), prob.cu_seqlens, block, topk)
        sels = [osel[(h, 0)][3][1] for h in range(hq)]
    else:
        rng = np.random.default_rng(91)
        own = np.arange(n) // block
        sels = []
        for h in range(hq):
            s = (rng.random((n, nB)) < 0.3) & (np.arange(nB)[None, :] <= own[:, None])
            s[rng.random(n) < 0.05] = False          # empty rows
            sels.append(s)
    log(f"case row selection {name}: n={n} hq={hq} hkv={prob.h_kv} d={prob.d} block={block} "
        f"picked {int(sum(s.sum() for s in sels))} row-blocks")
    _attn_case(name, prob, sels, block, dev)


def test_moba_batch2_and_strided_estimators():
    """Batch 2 (two seeded rows) for the MoBA gate and attention on its
    picks, and both alternative estimators on Q / K sliced from a fused
    [B, N, Hq + 2 Hkv, d] projection: their outputs equal those of the same
    values in contiguous tensors bit for bit."""
    dev = _dev()
    block, topk = 256, 3
    p1 = workloads.make_problem(2, n=2048, h_q=4, h_kv=1, seed=21)
    p2 = workloads.make_problem(2, n=2048, h_q=4, h_kv=1, seed=22)
    q = torch.cat([p1.q, p2.q])
    k = torch.cat([p1.k, p2.k])
    v = torch.cat([p1.v, p2.v])
    do = torch.cat([p1.do, p2.do])
    gq, gk, gv, gdo = q.to(dev), k.to(dev), v.to(dev), do.to(dev)
    gidx, gsc = vs.estimate_index_moba(gq, gk, block, topk, return_scores=True)
    torch.cuda.synchronize()
    words = gidx.row_mask.cpu().numpy()
    osels = []
    for b, p in enumerate((p1, p2)):
        q64, k64 = np64(p.q[0]), np64(p.k[0])
        osel, osc = oracle.estimate_index_moba(q64, k64, p.cu_seqlens, block, topk, return_scores=True)
        osels.append(osel)
        for h in range(4):
            check_gate(("b", b, h), q64[:, h], k64[:, 0], 2048, block, topk, gsc[b, h].cpu().numpy(), words[b, h],
                       osel[(h, 0)][3][1], osc[(h, 0)])
    # attention, batch 2, on the oracle's picks packed into row words
    ow = np.stack([[words_of(o[(h, 0)][3][1]) for h in range(4)] for o in osels]).astype(np.uint32)
    zeros = torch.zeros(2 * 4 + 1, dtype=torch.int32, device=dev)
    one = torch.zeros(1, dtype=torch.int32, device=dev)
    idx = vs.VsIndexT(zeros, one, zeros, one, 0, 0, row_mask=torch.from_numpy(ow.view(np.int32)).to(dev),
                      row_blk=block)
    o, lse = vs.sparse_attn_fwd(gq, gk, gv, idx)
    gdq, gdk, gdv = vs.sparse_attn_bwd(gq, gk, gv, o, gdo, lse, idx)
    torch.cuda.synchronize()
    pos = np.arange(2048)
    errs = []
    for b, p in enumerate((p1, p2)):
        osel = osels[b]
        q64, k64 = np64(p.q[0]), np64(p.k[0])
        v64, do64 = np64(p.v[0]), np64(p.do[0])
        O, L = oracle.attn_fwd_dense(q64, k64, v64, pos, pos, p.cu_seqlens, osel)
        D = oracle.bwd_delta(O, do64)
        dq, dk, dv = oracle.attn_bwd_dense(q64, k64, v64, do64, L, D, pos, pos, p.cu_seqlens, osel)
        bq, bk, bv = oracle.bwd_rounding_bounds(q64, k64, v64, do64, O, L, pos, pos, p.cu_seqlens, osel)
        errs += [check_close(f"b{b} O", O, np64(o[b]), "bf16", "o"),
                 check_close(f"b{b} LSE", L, lse[b].cpu().numpy().astype(np.float64), "bf16"),
                 check_close(f"b{b} dQ", dq, np64(gdq[b]), "bf16", "grad", bq),
                 check_close(f"b{b} dK", dk, np64(gdk[b]), "bf16", "grad", bk),
                 check_close(f"b{b} dV", dv, np64(gdv[b]), "bf16", "grad", bv)]
    errs = [e for e in errs if e]
    assert not errs, errs
    # fused projection: [B, N, Hq + 2 Hkv, d], Q / K / V as head slices
    fused = torch.cat([q, k, v], dim=2).to(dev)
    fq, fk = fused[:, :, :4], fused[:, :, 4:5]
    assert fq.stride(1) == 6 * 128 and not fq.is_contiguous()
    sidx, ssc = vs.estimate_index_moba(fq, fk, block, topk, return_scores=True)
    xidx, xcnt, xsc = vs.estimate_index_xattn(gq, gk, 0.9, return_scores=True)
    fxidx, fxcnt, fxsc = vs.estimate_index_xattn(fq, fk, 0.9, return_scores=True)
    torch.cuda.synchronize()
    assert torch.equal(sidx.row_mask, gidx.row_mask)
    own = torch.arange(2048, device=dev) // block
    early = torch.arange(2048 // block, device=dev)[None, :] < own[:, None]
    assert torch.equal(ssc[:, :, early], gsc[:, :, early])
    assert torch.equal(fxidx.blk_mask, xidx.blk_mask) and torch.equal(fxcnt, xcnt)
    tril = torch.tril(torch.ones(16, 16, dtype=torch.bool, device=dev))
    assert torch.equal(fxsc[:, :, tril], xsc[:, :, tril])
