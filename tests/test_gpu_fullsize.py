"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (one call each of the estimator, the forward and the
backward over the whole sequence; for the striped worker, the 32 ring-step
calls with the LSE merge and dQ accumulation).

The oracle cannot afford the whole problem, so it checks what it can compute
one piece at a time:
  * the estimator: every vertical / slash score and every selected list
    (the window is only 64 rows per segment);
  * O, LSE and dQ on sampled whole query blocks (first, second, a seeded
    middle one, the last two of each segment), all heads;
  * dK and dV exactly on the last key blocks of each segment: those keys are
    only seen by the rows of the last blocks, which the oracle computes in
    full;
and the rest through identities that hold at any size (MTraining §3.2 Eq. 1:
rowsum(dA * A) = D makes sum_m dS[n, m] = 0 and, with dQ = scale dS K and
dK = scale dS^T Q, the GQA group sums <dQ, Q> and <dK, K> agree).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from vs_cases import (check_close, check_xattn_row, index_parity, lists_for_gpu, log, np64,
                      pack_block_selection)

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(1200)]

vs = pytest.importorskip("dynamic_sparse_attention_amd")

TAIL = 3  # key blocks per segment whose dK / dV are checked exactly


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _window_q64(prob):
    """fp64 Q with only the estimator's window rows (last 64 of each segment) filled."""
    q = np.zeros((prob.n, prob.h_q, prob.d))
    for s in range(len(prob.cu_seqlens) - 1):
        e = prob.cu_seqlens[s + 1]
        a = max(prob.cu_seqlens[s], e - 64)
        q[a:e] = np64(prob.q[0, a:e])
    return q


def _estimate_and_check(prob, dev, gq, gk, cu):
    log(f"  oracle estimator (fp64, {prob.h_q} heads, {len(cu) - 1} segments)")
    oidx, osc = oracle.estimate_index(_window_q64(prob), np64(prob.k[0]), cu, prob.v_budget,
                                      prob.s_budget, prob.block, 64, return_scores=True)
    log("  GPU estimator")
    gidx, vsc, ssc = vs.estimate_index(gq, gk, prob.v_budget, prob.s_budget, cu, return_scores=True)
    torch.cuda.synchronize()
    index_parity(prob.name, oidx, osc, [(a.numpy(), b.numpy()) for a, b in gidx.lists()],
                 vsc[0].cpu().numpy(), ssc[0].cpu().numpy(), prob)
    return oidx


def _sample_blocks(nb, rng):
    mid = int(rng.integers(2, max(nb - 2, 3)))
    return sorted({b for b in (0, 1, mid, nb - 2, nb - 1) if 0 <= b < nb})


def _rows_of_blocks(starts_blocks):
    return np.concatenate([np.arange(64 * b, 64 * b + 64) for b in starts_blocks]).astype(np.int64)


def _mid_key_blocks(oidx, cu, heads, rng, per_seg=2):
    """Per segment, per_seg key blocks from the middle half of the segment in
    which no Q head of `heads` selected a vertical column: their keys are read
    only through selected block-diagonals, by the query blocks j + g, so the
    oracle gets their complete dK / dV from those rows alone."""
    out = []
    for s in range(len(cu) - 1):
        a, e = cu[s] // 64, cu[s + 1] // 64
        nb = e - a
        vert = set()
        for h in heads:
            vert.update((np.asarray(oidx[(h, s)][0]) // 64).tolist())
        cand = [b for b in range(a + nb // 4, a + (3 * nb) // 4) if b not in vert]
        if len(cand) < per_seg:
            cand = [b for b in range(a, e) if b not in vert]
        assert len(cand) >= per_seg, ("no key block free of verticals in segment", s)
        out.append(sorted(int(x) for x in rng.choice(cand, size=per_seg, replace=False)))
    return out


def _query_blocks_reading(oidx, cu, heads, seg, key_blocks):
    """Global query blocks j + g (g a selected block-diagonal of any head in
    `heads`) that read the given global key blocks of segment seg."""
    a, e = cu[seg] // 64, cu[seg + 1] // 64
    qb = set()
    for h in heads:
        for g in np.asarray(oidx[(h, seg)][1]).tolist():
            for j in key_blocks:
                if j + g < e:
                    qb.add(j + g)
    return sorted(qb)


def _group_index(oidx, heads, n_seg):
    """The index of the Q heads `heads` (one KV group), renumbered 0..len-1."""
    return {(i, s): oidx[(h, s)] for i, h in enumerate(heads) for s in range(n_seg)}


def _check_mid_key_blocks(name, prob, oidx, rows_of, dk, dv, key_pos, grp, rng, per_seg=2):
    """Element-wise dK / dV of mid-sequence key blocks of KV group grp against
    the oracle, computed from every row that reads them.

    The key blocks hold no vertical column of the group's heads (see
    _mid_key_blocks), so rows_of(query blocks j + g) are all their readers;
    rows_of maps global query blocks to the global rows this call holds (all
    rows, or a striped worker's).  dk / dv [keys, d] are the GPU's gradients of
    the global key positions key_pos (ascending) of group grp."""
    cu = prob.cu_seqlens
    n_seg = len(cu) - 1
    G = prob.h_q // prob.h_kv
    heads = list(range(grp * G, (grp + 1) * G))
    kblocks = _mid_key_blocks(oidx, cu, heads, rng, per_seg)
    qblocks = sorted(set().union(*[_query_blocks_reading(oidx, cu, heads, s, kb)
                                   for s, kb in enumerate(kblocks)]))
    rows = rows_of(qblocks)
    keys = np.concatenate([np.arange(64 * b, 64 * b + 64) for kb in kblocks for b in kb])
    log(f"  {name}: dK / dV of key blocks {kblocks} (group {grp}), from {len(rows)} rows")
    gidx = _group_index(oidx, heads, n_seg)
    k64 = np64(prob.k[0, :, grp:grp + 1])
    v64 = np64(prob.v[0, :, grp:grp + 1])
    cols = np.arange(prob.n)
    q_r, do_r = np64(prob.q[0, rows][:, heads]), np64(prob.do[0, rows][:, heads])
    O, L = oracle.attn_fwd_support(q_r, k64, v64, rows, cols, cu, gidx)
    D = oracle.bwd_delta(O, do_r)
    _, dk_o, dv_o = oracle.attn_bwd_support(q_r, k64, v64, do_r, L, D, rows, cols, cu, gidx)
    _, bk, bv = oracle.bwd_rounding_bounds(q_r, k64, v64, do_r, O, L, rows, cols, cu, gidx, support=True)
    sel = np.searchsorted(key_pos, keys)
    assert np.array_equal(key_pos[sel], keys)
    return [check_close(f"{name} dK (mid keys, group {grp})", dk_o[keys, 0], dk[sel], "bf16", "grad", bk[keys, 0]),
            check_close(f"{name} dV (mid keys, group {grp})", dv_o[keys, 0], dv[sel], "bf16", "grad", bv[keys, 0])]


def _kernel_split_checks(prob, oidx, gq, gk, gv, gdo, dev, rng, verticals=True):
    """The two dK / dV kernels at full size, each on an index of its own part.

    Slash-only index (the estimated block-diagonals, no verticals): every key
    is read only through block-diagonals, so mid-sequence key blocks of each
    segment are compared element by element from the rows j + g that read
    them; with 8 heads x k_g diagonals a key block's tile list is emptied and
    refilled several times.  Two such blocks with one document, one per
    document with several.  Verticals-only index (every 8th estimated column,
    no block-diagonals; when `verticals`): dK / dV of every key of KV group 0,
    from the oracle over all rows of the group's heads."""
    cu = prob.cu_seqlens
    n_seg = len(cu) - 1
    errs = []
    empty = np.zeros(0, np.int64)
    sl = {key: (empty, val[1]) for key, val in oidx.items()}
    idx = vs.index_from_lists(lists_for_gpu(sl, prob.h_q, n_seg), dev)
    log("  GPU forward + backward on the slash-only index")
    o, lse = vs.sparse_attn_fwd(gq, gk, gv, idx, cu)
    _, dk, dv = vs.sparse_attn_bwd(gq, gk, gv, o, gdo, lse, idx, cu_seqlens=cu)
    torch.cuda.synchronize()
    errs += _check_mid_key_blocks("slash-only", prob, sl, _rows_of_blocks, np64(dk[0, :, 0]),
                                  np64(dv[0, :, 0]), np.arange(prob.n), 0, rng, 2 if n_seg == 1 else 1)
    del o, lse, dk, dv
    if not verticals:
        return errs
    vt = {key: (val[0][::8], empty) for key, val in oidx.items()}
    idx = vs.index_from_lists(lists_for_gpu(vt, prob.h_q, n_seg), dev)
    log("  GPU forward + backward on the verticals-only index")
    o, lse = vs.sparse_attn_fwd(gq, gk, gv, idx, cu)
    _, dk, dv = vs.sparse_attn_bwd(gq, gk, gv, o, gdo, lse, idx, cu_seqlens=cu)
    torch.cuda.synchronize()
    G = prob.h_q // prob.h_kv
    heads = list(range(G))
    log(f"  oracle on all {prob.n} rows of group 0 (verticals-only index)")
    rows = np.arange(prob.n)
    q_r, do_r = np64(prob.q[0][:, heads]), np64(prob.do[0][:, heads])
    k64, v64 = np64(prob.k[0, :, 0:1]), np64(prob.v[0, :, 0:1])
    gidx = _group_index(vt, heads, n_seg)
    O, L = oracle.attn_fwd_support(q_r, k64, v64, rows, rows, cu, gidx)
    D = oracle.bwd_delta(O, do_r)
    _, dk_o, dv_o = oracle.attn_bwd_support(q_r, k64, v64, do_r, L, D, rows, rows, cu, gidx)
    _, bk, bv = oracle.bwd_rounding_bounds(q_r, k64, v64, do_r, O, L, rows, rows, cu, gidx, support=True)
    errs += [check_close("verticals-only dK (all keys, group 0)", dk_o[:, 0], np64(dk[0, :, 0]), "bf16", "grad", bk[:, 0]),
             check_close("verticals-only dV (all keys, group 0)", dv_o[:, 0], np64(dv[0, :, 0]), "bf16", "grad", bv[:, 0])]
    return errs


def _dv_identity(name, dv, v, o, do, h_q, h_kv):
    """sum_{h in group} sum_n delta_h[n] == <dV_g, V_g> per KV group, with
    delta = rowsum(dO * O) from the GPU's own O (fp64 sums of GPU tensors).

    dV = A^T dO gives <dV, V> = sum_n <dO_n, sum_m A[n, m] V_m> = sum_n <dO_n, O_n>
    (MTraining §3.2 Eq. 1: rowsum(dA * A) = rowsum(dO * O)); both sides use
    bf16-rounded probabilities, so they agree to a small fraction of
    sum |dO| |O|."""
    errs = []
    for g in range(h_kv):
        hs = [h for h in range(h_q) if h * h_kv // h_q == g]
        rhs = sum(float((do[:, h].double() * o[:, h].double()).sum()) for h in hs)
        mag = sum(float((do[:, h].double() * o[:, h].double()).abs().sum()) for h in hs)
        lhs = float((dv[:, g].double() * v[:, g].double()).sum())
        rel = abs(lhs - rhs) / max(mag, 1e-30)
        log(f"  {name} group {g}: <dV,V>={lhs:.6e} sum delta={rhs:.6e} |diff|/sum|dO*O|={rel:.2e}")
        if rel > 1e-4:
            errs.append(f"{name} group {g}: dV identity off by {rel:.2e}")
    return errs


def _group_identity(name, dq, q, dk, k, h_q, h_kv):
    """sum_{h in group} <dQ_h, Q_h> == <dK_g, K_g> per KV group (fp64 sums of the GPU tensors).

    Both sides are scale * sum dS[n, m] (q_n . k_m) over the support; the two
    kernels round their own fp32 dS to bf16 and accumulate in a different
    order, so they agree to a small fraction of sum |dQ| |Q|.
    """
    errs = []
    for g in range(h_kv):
        hs = [h for h in range(h_q) if h * h_kv // h_q == g]
        lhs = sum(float((dq[:, h].double() * q[:, h].double()).sum()) for h in hs)
        mag = sum(float((dq[:, h].double().abs() * q[:, h].double().abs()).sum()) for h in hs)
        rhs = float((dk[:, g].double() * k[:, g].double()).sum())
        rel = abs(lhs - rhs) / max(mag, 1e-30)
        log(f"  {name} group {g}: <dQ,Q>={lhs:.6e} <dK,K>={rhs:.6e} |diff|/sum|dQ||Q|={rel:.2e}")
        if rel > 1e-4:
            errs.append(f"{name} group {g}: identity off by {rel:.2e}")
    return errs


@pytest.mark.parametrize("wid", [2, 3, 5])
def test_fullsize_contiguous(wid):
    dev = _dev()
    log(f"full-size workload {wid}: drawing inputs")
    prob = workloads.make_problem(wid)
    cu = prob.cu_seqlens
    n_seg = len(cu) - 1
    log(f"  {prob.name}: n={prob.n} hq={prob.h_q} hkv={prob.h_kv} d={prob.d} segments={n_seg}")
    gq, gk, gv, gdo = (t.to(dev) for t in (prob.q, prob.k, prob.v, prob.do))
    oidx = _estimate_and_check(prob, dev, gq, gk, cu)

    log("  GPU forward + backward (whole sequence)")
    idx = vs.index_from_lists(lists_for_gpu(oidx, prob.h_q, n_seg), dev)
    o, lse = vs.sparse_attn_fwd(gq, gk, gv, idx, cu)
    dq, dk, dv = vs.sparse_attn_bwd(gq, gk, gv, o, gdo, lse, idx, cu_seqlens=cu)
    torch.cuda.synchronize()

    k64, v64 = np64(prob.k[0]), np64(prob.v[0])
    cols = np.arange(prob.n)
    rng = np.random.default_rng(prob.seed)
    errs = []

    # sampled query blocks: O, LSE, dQ (with several segments, one block of
    # each, cycling through first / last / a seeded middle one)
    blocks = []
    for s in range(n_seg):
        a, nb = cu[s] // 64, (cu[s + 1] - cu[s]) // 64
        pick = _sample_blocks(nb, rng)
        if n_seg > 1:
            pick = [(pick[0], pick[-1], pick[len(pick) // 2])[s % 3]]
        blocks += [a + b for b in pick]
    rows = _rows_of_blocks(blocks)
    log(f"  oracle on {len(blocks)} sampled query blocks")
    q_r, do_r = np64(prob.q[0, rows]), np64(prob.do[0, rows])
    O, L = oracle.attn_fwd_support(q_r, k64, v64, rows, cols, cu, oidx)
    D = oracle.bwd_delta(O, do_r)
    dq_o, _, _ = oracle.attn_bwd_support(q_r, k64, v64, do_r, L, D, rows, cols, cu, oidx)
    bq, _, _ = oracle.bwd_rounding_bounds(q_r, k64, v64, do_r, O, L, rows, cols, cu, oidx, support=True)
    rt = torch.from_numpy(rows).to(dev)
    errs += [check_close("O (sampled)", O, np64(o[0, rt]), prob.dtype, "o"),
             check_close("LSE (sampled)", L, np64(lse[0][:, rt]), prob.dtype),
             check_close("dQ (sampled)", dq_o, np64(dq[0, rt]), prob.dtype, "grad", bq)]

    # the last TAIL key blocks of a segment: only its last TAIL query blocks
    # see them (first and last segment when there are several)
    tail_blocks = []
    for s in sorted({0, n_seg - 1}):
        b1 = cu[s + 1] // 64
        tail_blocks += list(range(max(cu[s] // 64, b1 - TAIL), b1))
    rows = _rows_of_blocks(tail_blocks)
    log(f"  oracle on the last {TAIL} blocks of each segment ({len(rows)} rows)")
    q_r, do_r = np64(prob.q[0, rows]), np64(prob.do[0, rows])
    O, L = oracle.attn_fwd_support(q_r, k64, v64, rows, cols, cu, oidx)
    D = oracle.bwd_delta(O, do_r)
    _, dk_o, dv_o = oracle.attn_bwd_support(q_r, k64, v64, do_r, L, D, rows, cols, cu, oidx)
    _, bk, bv = oracle.bwd_rounding_bounds(q_r, k64, v64, do_r, O, L, rows, cols, cu, oidx, support=True)
    rt = torch.from_numpy(rows).to(dev)
    errs += [check_close("dK (tail keys)", dk_o[rows], np64(dk[0, rt]), prob.dtype, "grad", bk[rows]),
             check_close("dV (tail keys)", dv_o[rows], np64(dv[0, rt]), prob.dtype, "grad", bv[rows])]

    errs += _group_identity(prob.name, dq[0], gq[0], dk[0], gk[0], prob.h_q, prob.h_kv)
    errs += _dv_identity(prob.name, dv[0], gv[0], o[0], gdo[0], prob.h_q, prob.h_kv)
    del o, lse, dq, dk, dv
    errs += _kernel_split_checks(prob, oidx, gq, gk, gv, gdo, dev, rng, verticals=(wid == 3))
    errs = [e for e in errs if e]
    assert not errs, errs


def test_fullsize_striped_worker():
    """Worker 0 of 32 on the 524288-token sequence: 32 forward calls merging
    into the running result (fused; the same with lse_merge must agree), then
    32 backward calls accumulating dQ (Algorithm 2 of the MTraining paper note,
    run as one worker's share)."""
    dev = _dev()
    log("full-size workload 4: drawing inputs")
    prob = workloads.make_problem(4)
    W, w = prob.stripe_world, prob.stripe_rank
    cu = prob.cu_seqlens
    log(f"  {prob.name}: n={prob.n} world={W} rank={w}")
    gq_all, gk_all = prob.q.to(dev), prob.k.to(dev)
    oidx = _estimate_and_check(prob, dev, gq_all, gk_all, cu)
    del gq_all, gk_all
    idx = vs.index_from_lists(lists_for_gpu(oidx, prob.h_q, 1), dev)

    rows_all = workloads.stripe_positions(prob.n, W, w).numpy()
    gq = workloads.stripe_rows(prob.q, W, w).to(dev)
    gdo = workloads.stripe_rows(prob.do, W, w).to(dev)
    nq = gq.shape[1]
    chunks = []
    for t in range(W):
        u = (w - t) % W
        chunks.append((u, workloads.stripe_rows(prob.k, W, u).to(dev),
                       workloads.stripe_rows(prob.v, W, u).to(dev)))
    log(f"  GPU: {W} forward calls with the merge fused, {W} forward calls + lse_merge, {W} backward calls")
    acc_o = torch.zeros((1, nq, prob.h_q, prob.d), device=dev)
    acc_l = torch.full((1, prob.h_q, nq), -float("inf"), device=dev)
    for u, gk, gv in chunks:
        vs.sparse_attn_fwd(gq, gk, gv, idx, stripe=(W, w, u), out=acc_o, lse=acc_l, merge=True)
    sep_o = torch.zeros_like(acc_o)
    sep_l = torch.full_like(acc_l, -float("inf"))
    for u, gk, gv in chunks:
        o, l = vs.sparse_attn_fwd(gq, gk, gv, idx, stripe=(W, w, u), o_f32=True)
        vs.lse_merge(sep_o, sep_l, o, l)
    del o, l
    torch.cuda.synchronize()
    # the fused and the separate merge do the same fp32 arithmetic up to one rounding
    assert torch.allclose(acc_o, sep_o, rtol=1e-5, atol=1e-6)
    fin = torch.isfinite(sep_l)
    assert torch.equal(fin, torch.isfinite(acc_l)) and torch.allclose(acc_l[fin], sep_l[fin], rtol=1e-6, atol=1e-5)
    del sep_o, sep_l
    delta = vs.attn_bwd_delta(acc_o, gdo)
    dq = torch.zeros((1, nq, prob.h_q, prob.d), device=dev)
    k64, v64 = np64(prob.k[0]), np64(prob.v[0])
    cols = np.arange(prob.n)
    nqb = nq // 64
    # worker rows of its last two local blocks are the only ones that see keys
    # in global blocks after the worker's third-to-last block
    tail_local = [nqb - 2, nqb - 1]
    first_key_blk = rows_all[64 * (nqb - 3)] // 64 + 1
    dk_tail, dv_tail, key_tail = [], [], []
    # mid-sequence key blocks checked below: no vertical of group 0 in them
    G = prob.h_q // prob.h_kv
    rng_mid = np.random.default_rng(prob.seed + 1)
    mid_blocks = _mid_key_blocks(oidx, cu, list(range(G)), rng_mid)[0]
    mid_keys = np.concatenate([np.arange(64 * b, 64 * b + 64) for b in mid_blocks])
    dk_mid, dv_mid, key_mid = [], [], []
    lhs_k = np.zeros(prob.h_kv)
    lhs_v = np.zeros(prob.h_kv)
    for u, gk, gv in chunks:
        _, dk, dv = vs.sparse_attn_bwd(gq, gk, gv, None, gdo, acc_l, idx, delta=delta, dq=dq,
                                       stripe=(W, w, u), accumulate=True)
        kpos = workloads.stripe_positions(prob.n, W, u).numpy()
        sel = np.nonzero(kpos // 64 >= first_key_blk)[0]
        st = torch.from_numpy(sel).to(dev)
        dk_tail.append(np64(dk[0, st]))
        dv_tail.append(np64(dv[0, st]))
        key_tail.append(kpos[sel])
        msel = np.nonzero(np.isin(kpos, mid_keys))[0]
        if msel.size:
            mt = torch.from_numpy(msel).to(dev)
            dk_mid.append(np64(dk[0, mt, 0]))
            dv_mid.append(np64(dv[0, mt, 0]))
            key_mid.append(kpos[msel])
        for g in range(prob.h_kv):
            lhs_k[g] += float((dk[0, :, g].double() * gk[0, :, g].double()).sum())
            lhs_v[g] += float((dv[0, :, g].double() * gv[0, :, g].double()).sum())
    torch.cuda.synchronize()
    dk_tail, dv_tail, key_tail = np.concatenate(dk_tail), np.concatenate(dv_tail), np.concatenate(key_tail)

    errs = []
    rng = np.random.default_rng(prob.seed)
    lblocks = _sample_blocks(nqb, rng)
    lrows = _rows_of_blocks(lblocks)
    rows = rows_all[lrows]
    log(f"  oracle on worker blocks {lblocks}")
    q_r, do_r = np64(prob.q[0, rows]), np64(prob.do[0, rows])
    O, L = oracle.attn_fwd_support(q_r, k64, v64, rows, cols, cu, oidx)
    D = oracle.bwd_delta(O, do_r)
    dq_o, _, _ = oracle.attn_bwd_support(q_r, k64, v64, do_r, L, D, rows, cols, cu, oidx)
    bq, _, _ = oracle.bwd_rounding_bounds(q_r, k64, v64, do_r, O, L, rows, cols, cu, oidx,
                                          u_o=2.0 ** -24, support=True)
    lt = torch.from_numpy(lrows).to(dev)
    errs += [check_close("merged O (sampled)", O, np64(acc_o[0, lt]), "bf16", "o"),
             check_close("merged LSE (sampled)", L, np64(acc_l[0][:, lt]), "bf16"),
             check_close("accumulated dQ (sampled)", dq_o, np64(dq[0, lt]), "bf16", "grad", bq)]

    lrows = _rows_of_blocks(tail_local)
    rows = rows_all[lrows]
    log(f"  oracle on worker blocks {tail_local}: dK / dV of global key blocks >= {first_key_blk}")
    q_r, do_r = np64(prob.q[0, rows]), np64(prob.do[0, rows])
    O, L = oracle.attn_fwd_support(q_r, k64, v64, rows, cols, cu, oidx)
    D = oracle.bwd_delta(O, do_r)
    _, dk_o, dv_o = oracle.attn_bwd_support(q_r, k64, v64, do_r, L, D, rows, cols, cu, oidx)
    _, bk, bv = oracle.bwd_rounding_bounds(q_r, k64, v64, do_r, O, L, rows, cols, cu, oidx,
                                           u_o=2.0 ** -24, support=True)
    errs += [check_close("dK share (tail keys)", dk_o[key_tail], dk_tail, "bf16", "grad", bk[key_tail]),
             check_close("dV share (tail keys)", dv_o[key_tail], dv_tail, "bf16", "grad", bv[key_tail])]

    # mid-sequence key blocks: every worker row that reads them (the worker's
    # rows among the query blocks j + g)
    dk_mid, dv_mid, key_mid = np.concatenate(dk_mid), np.concatenate(dv_mid), np.concatenate(key_mid)
    order = np.argsort(key_mid)
    worker_blocks = set((rows_all[::64] // 64).tolist())

    def worker_rows(qblocks):
        mine = [b for b in qblocks if b in worker_blocks]
        return _rows_of_blocks(mine) if mine else np.zeros(0, np.int64)

    errs += _check_mid_key_blocks("ring worker", prob, oidx, worker_rows, dk_mid[order], dv_mid[order],
                                  key_mid[order], 0, np.random.default_rng(prob.seed + 1))
    for g in range(prob.h_kv):
        hs = [h for h in range(prob.h_q) if h * prob.h_kv // prob.h_q == g]
        lhs = sum(float((dq[0, :, h].double() * gq[0, :, h].double()).sum()) for h in hs)
        mag = sum(float((dq[0, :, h].double().abs() * gq[0, :, h].double().abs()).sum()) for h in hs)
        rel = abs(lhs - lhs_k[g]) / max(mag, 1e-30)
        log(f"  ring group {g}: <dQ,Q>={lhs:.6e} sum_u <dK_u,K_u>={lhs_k[g]:.6e} rel={rel:.2e}")
        if rel > 1e-4:
            errs.append(f"ring group {g}: identity off by {rel:.2e}")
        rhs = sum(float((gdo[0, :, h].double() * acc_o[0, :, h].double()).sum()) for h in hs)
        magv = sum(float((gdo[0, :, h].double() * acc_o[0, :, h].double()).abs().sum()) for h in hs)
        relv = abs(lhs_v[g] - rhs) / max(magv, 1e-30)
        log(f"  ring group {g}: sum_u <dV_u,V_u>={lhs_v[g]:.6e} sum delta={rhs:.6e} rel={relv:.2e}")
        if relv > 1e-4:
            errs.append(f"ring group {g}: dV identity off by {relv:.2e}")
    errs = [e for e in errs if e]
    assert not errs, errs


def test_fullsize_xattn():
    """XAttention (block 128, stride 16, threshold 0.9) at N = 131072 on
    workload 3's inputs, in bench.py --estimator xattn's launch configuration.

    Estimator: for every Q head and query block, the device's count and
    bitmap equal the integer decision on its own scores; for one Q head per
    KV group, every block score against the oracle's and every selection
    against the oracle's (certified near ties allowed).  Attention on a block
    selection: those two heads take the oracle's selection, the others seeded
    random selections of 90 % of the causal blocks (host-drawn); O, LSE and
    dQ of sampled query blocks of the two heads against the oracle, dK and
    dV of the last key blocks (read only by the last query blocks) against
    the oracle over all heads, and the group identities."""
    dev = _dev()
    thr = 0.9
    log("full-size XAttention: drawing inputs (workload 3)")
    prob = workloads.make_problem(3)
    n, hq, hkv = prob.n, prob.h_q, prob.h_kv
    nI = n // 128
    G = hq // hkv
    cu = prob.cu_seqlens
    gq, gk, gv, gdo = (t.to(dev) for t in (prob.q, prob.k, prob.v, prob.do))
    log("  GPU estimator")
    gidx, gcnt, gsc = vs.estimate_index_xattn(gq, gk, thr, return_scores=True)
    torch.cuda.synchronize()
    gsel = gidx.block_selection(n).numpy()
    gcnt = gcnt[0].cpu().numpy()
    gsc = gsc[0].cpu().numpy()
    del gidx
    # every head: the device's decision on its own scores (oracle count unknown: pass its own)
    from vs_cases import xattn_count_int
    for h in range(hq):
        for I in range(nI):
            kk, order = xattn_count_int(gsc[h, I, :I + 1], thr)
            assert gcnt[h, I] == kk, (h, I, int(gcnt[h, I]), kk)
            want = np.zeros(nI, bool)
            want[order[:kk]] = True
            assert np.array_equal(gsel[h, I], want), (h, I)
    heads = [grp * G for grp in range(hkv)]
    q64, k64 = np64(prob.q[0]), np64(prob.k[0])
    osel = {}
    for h in heads:
        log(f"  oracle block scores, head {h}")
        out, osc, ocnt = oracle.estimate_index_xattn(q64[:, h:h + 1], k64[:, h // G:h // G + 1], cu, 128, 16,
                                                     thr, return_scores=True)
        worst, flips, swaps = 0.0, 0, 0
        for I in range(nI):
            e, f, w, _ = check_xattn_row((h, I), osc[(0, 0)][I, :I + 1], gsc[h, I, :I + 1], gsel[h, I],
                                         gcnt[h, I], int(ocnt[(0, 0)][I]), thr)
            worst, flips, swaps = max(worst, e), flips + f, swaps + w
        osel[h] = out[(0, 0)][2][1]
        log(f"  head {h}: score err/(1+s) max {worst:.2e}, flips {flips}, swaps {swaps}; "
            f"{int(osel[h].sum())} of {nI * (nI + 1) // 2} causal blocks selected")
    del gsc, gsel

    rng = np.random.default_rng(prob.seed + 77)
    tril = np.tril(np.ones((nI, nI), bool))
    sels = [osel[h] if h in osel else (rng.random((nI, nI)) < 0.9) & tril for h in range(hq)]
    mask = pack_block_selection(sels, nI).to(dev)
    zeros = torch.zeros(hq + 1, dtype=torch.int32, device=dev)
    one = torch.zeros(1, dtype=torch.int32, device=dev)
    idx = vs.VsIndexT(zeros, one, zeros, one, 0, 0, mask, 128)
    log("  GPU forward + backward on the block selection")
    o, lse = vs.sparse_attn_fwd(gq, gk, gv, idx)
    dq, dk, dv = vs.sparse_attn_bwd(gq, gk, gv, o, gdo, lse, idx)
    torch.cuda.synchronize()
    empty = np.zeros(0, np.int64)
    cols = np.arange(n)
    v64 = np64(prob.v[0])
    errs = []
    # O, LSE, dQ of sampled query blocks of the two oracle-selected heads
    blocks = _sample_blocks(n // 64, np.random.default_rng(prob.seed))
    rows = _rows_of_blocks(blocks)
    sub = {(i, 0): (empty, empty, (128, sels[h])) for i, h in enumerate(heads)}
    log(f"  oracle on {len(blocks)} sampled query blocks of heads {heads}")
    q_r, do_r = q64[rows][:, heads], np64(prob.do[0, rows][:, heads])
    O, L = oracle.attn_fwd_support(q_r, k64, v64, rows, cols, cu, sub)
    D = oracle.bwd_delta(O, do_r)
    dq_o, _, _ = oracle.attn_bwd_support(q_r, k64, v64, do_r, L, D, rows, cols, cu, sub)
    bq, _, _ = oracle.bwd_rounding_bounds(q_r, k64, v64, do_r, O, L, rows, cols, cu, sub, support=True)
    rt = torch.from_numpy(rows).to(dev)
    ht = torch.tensor(heads, device=dev)
    errs += [check_close("xattn O (sampled)", O, np64(o[0, rt][:, ht]), "bf16", "o"),
             check_close("xattn LSE (sampled)", L, np64(lse[0][ht][:, rt]), "bf16"),
             check_close("xattn dQ (sampled)", dq_o, np64(dq[0, rt][:, ht]), "bf16", "grad", bq)]
    # dK / dV of the last TAIL key blocks from the last TAIL query blocks, all heads
    rows = _rows_of_blocks(range(n // 64 - TAIL, n // 64))
    full = {(h, 0): (empty, empty, (128, sels[h])) for h in range(hq)}
    log(f"  oracle on the last {TAIL} query blocks, all heads")
    q_r, do_r = q64[rows], np64(prob.do[0, rows])
    O, L = oracle.attn_fwd_support(q_r, k64, v64, rows, cols, cu, full)
    D = oracle.bwd_delta(O, do_r)
    _, dk_o, dv_o = oracle.attn_bwd_support(q_r, k64, v64, do_r, L, D, rows, cols, cu, full)
    _, bk, bv = oracle.bwd_rounding_bounds(q_r, k64, v64, do_r, O, L, rows, cols, cu, full, support=True)
    rt = torch.from_numpy(rows).to(dev)
    errs += [check_close("xattn dK (tail keys)", dk_o[rows], np64(dk[0, rt]), "bf16", "grad", bk[rows]),
             check_close("xattn dV (tail keys)", dv_o[rows], np64(dv[0, rt]), "bf16", "grad", bv[rows])]
    errs += _group_identity("xattn", dq[0], gq[0], dk[0], gk[0], hq, hkv)
    errs += _dv_identity("xattn", dv[0], gv[0], o[0], gdo[0], hq, hkv)
    errs = [e for e in errs if e]
    assert not errs, errs


def test_fullsize_moba():
    """MoBA (block 4096, top-12) at N = 131072 on workload 3's inputs, in
    bench.py --estimator moba's launch configuration.

    Gate: for every Q head and row, the device's word equals the selection
    recomputed from its own fp32 scores; for one Q head per KV group, the
    scores and words against the oracle (certified near ties allowed).
    Attention on the per-row selection: those two heads take the oracle's
    selection, the others seeded ones (the own block and 11 random earlier
    blocks); O, LSE and dQ of sampled query blocks of the two heads, dK and dV
    of the last key blocks from all heads, and the group identities."""
    from test_gpu_moba import SCORE_REL, check_gate, words_of
    dev = _dev()
    block, topk = 4096, 12
    log("full-size MoBA: drawing inputs (workload 3)")
    prob = workloads.make_problem(3)
    n, hq, hkv = prob.n, prob.h_q, prob.h_kv
    G = hq // hkv
    nB = n // block
    cu = prob.cu_seqlens
    gq, gk, gv, gdo = (t.to(dev) for t in (prob.q, prob.k, prob.v, prob.do))
    log("  GPU gate")
    gidx, gsc = vs.estimate_index_moba(gq, gk, block, topk, return_scores=True)
    torch.cuda.synchronize()
    words = gidx.row_mask[0].cpu().numpy().astype(np.int64) & 0xFFFFFFFF
    gsc = gsc[0].cpu().numpy()
    del gidx
    own = np.arange(n) // block
    J = np.arange(nB)
    earlier = J[None, :] < own[:, None]
    for h in range(hq):
        s = gsc[h]
        # rank of J among the row's earlier blocks (higher first, ties to the lower index)
        beats = (s[:, :, None] > s[:, None, :]) | ((s[:, :, None] == s[:, None, :]) & (J[:, None] < J[None, :]))
        rank = (beats & earlier[:, :, None]).sum(axis=1)
        pick = (earlier & (rank < topk - 1)) | (J[None, :] == own[:, None])
        assert np.array_equal(words[h], words_of(pick)), h
    heads = [grp * G for grp in range(hkv)]
    q64, k64 = np64(prob.q[0]), np64(prob.k[0])
    sels = {}
    for h in heads:
        log(f"  oracle gate, head {h}")
        out, osc = oracle.estimate_index_moba(q64[:, h:h + 1], k64[:, h // G:h // G + 1], cu, block, topk,
                                              return_scores=True)
        sels[h] = out[(0, 0)][3][1]
        worst, flips = check_gate(("moba", h), q64[:, h], k64[:, h // G], n, block, topk, gsc[h], words[h],
                                  sels[h], osc[(0, 0)])
        log(f"  head {h}: score err/bound max {worst:.2e}, certified near-tie rows {flips}; "
            f"{int(sels[h].sum())} row-blocks picked")
    del gsc
    rng = np.random.default_rng(prob.seed + 91)
    allsel = []
    for h in range(hq):
        if h in sels:
            allsel.append(sels[h])
            continue
        s = np.zeros((n, nB), bool)
        s[np.arange(n), own] = True
        for b_ in range(1, nB):
            rows = np.arange(b_ * block, (b_ + 1) * block)
            r = rng.random((rows.size, b_)).argsort(axis=1)[:, :topk - 1]
            s[rows[:, None], r] = True
        allsel.append(s)
    w = np.stack([words_of(s) for s in allsel]).astype(np.uint32).view(np.int32)
    zeros = torch.zeros(hq + 1, dtype=torch.int32, device=dev)
    one = torch.zeros(1, dtype=torch.int32, device=dev)
    idx = vs.VsIndexT(zeros, one, zeros, one, 0, 0,
                      row_mask=torch.from_numpy(w).reshape(1, hq, n).to(dev), row_blk=block)
    log("  GPU forward + backward on the per-row selection")
    o, lse = vs.sparse_attn_fwd(gq, gk, gv, idx)
    dq, dk, dv = vs.sparse_attn_bwd(gq, gk, gv, o, gdo, lse, idx)
    torch.cuda.synchronize()
    empty = np.zeros(0, np.int64)
    cols = np.arange(n)
    v64 = np64(prob.v[0])
    errs = []
    blocks = _sample_blocks(n // 64, np.random.default_rng(prob.seed))
    rows = _rows_of_blocks(blocks)
    sub = {(i, 0): (empty, empty, None, (block, allsel[h])) for i, h in enumerate(heads)}
    log(f"  oracle on {len(blocks)} sampled query blocks of heads {heads}")
    q_r, do_r = q64[rows][:, heads], np64(prob.do[0, rows][:, heads])
    O, L = oracle.attn_fwd_support(q_r, k64, v64, rows, cols, cu, sub)
    D = oracle.bwd_delta(O, do_r)
    dq_o, _, _ = oracle.attn_bwd_support(q_r, k64, v64, do_r, L, D, rows, cols, cu, sub)
    bq, _, _ = oracle.bwd_rounding_bounds(q_r, k64, v64, do_r, O, L, rows, cols, cu, sub, support=True)
    rt = torch.from_numpy(rows).to(dev)
    ht = torch.tensor(heads, device=dev)
    errs += [check_close("moba O (sampled)", O, np64(o[0, rt][:, ht]), "bf16", "o"),
             check_close("moba LSE (sampled)", L, np64(lse[0][ht][:, rt]), "bf16"),
             check_close("moba dQ (sampled)", dq_o, np64(dq[0, rt][:, ht]), "bf16", "grad", bq)]
    rows = _rows_of_blocks(range(n // 64 - TAIL, n // 64))
    full = {(h, 0): (empty, empty, None, (block, allsel[h])) for h in range(hq)}
    log(f"  oracle on the last {TAIL} query blocks, all heads")
    q_r, do_r = q64[rows], np64(prob.do[0, rows])
    O, L = oracle.attn_fwd_support(q_r, k64, v64, rows, cols, cu, full)
    D = oracle.bwd_delta(O, do_r)
    _, dk_o, dv_o = oracle.attn_bwd_support(q_r, k64, v64, do_r, L, D, rows, cols, cu, full)
    _, bk, bv = oracle.bwd_rounding_bounds(q_r, k64, v64, do_r, O, L, rows, cols, cu, full, support=True)
    rt = torch.from_numpy(rows).to(dev)
    errs += [check_close("moba dK (tail keys)", dk_o[rows], np64(dk[0, rt]), "bf16", "grad", bk[rows]),
             check_close("moba dV (tail keys)", dv_o[rows], np64(dv[0, rt]), "bf16", "grad", bv[rows])]
    errs += _group_identity("moba", dq[0], gq[0], dk[0], gk[0], hq, hkv)
    errs += _dv_identity("moba", dv[0], gv[0], o[0], gdo[0], hq, hkv)
    errs = [e for e in errs if e]
    assert not errs, errs
