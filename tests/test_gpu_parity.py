"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Small and medium problems are compared element by element; every case spans
several 64-row/64-key tiles, ragged vertical tiles (budgets that are not a
multiple of 64) and, where named, packed documents or block striping.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from vs_cases import assert_close, check_close, index_parity, lists_for_gpu, log, np64, oracle_index

pytestmark = pytest.mark.gpu

vs = pytest.importorskip("dynamic_sparse_attention_amd")


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


CASES = {
    # name: make_problem kwargs
    "w1-full-fp32": dict(wid=1),
    "w2-n4096": dict(wid=2, n=4096, v_budget=300, s_budget=1024),
    "w2-n2048-d64": dict(wid=2, n=2048, h_q=4, h_kv=1, d=64, v_budget=100, s_budget=300),
    "w5-n8192-docs": dict(wid=5, n=8192, n_docs=4),
    "dense-bf16": dict(wid=2, n=1024, h_q=2, h_kv=1, v_budget=0, s_budget=1024),
    "verticals-only": dict(wid=2, n=2048, h_q=2, h_kv=1, v_budget=333, s_budget=0),
    "empty": dict(wid=2, n=1024, h_q=2, h_kv=1, v_budget=0, s_budget=0),
    "w1-fp32-d128-gqa": dict(wid=1, n=2048, h_q=4, h_kv=2, d=128, v_budget=200, s_budget=256),
    # three Q heads per KV head: the bf16 kernels that serve one head per workgroup
    "w2-gqa3-odd": dict(wid=2, n=3072, h_q=3, h_kv=1, v_budget=250, s_budget=700),
    # 32 Q heads on one KV head: the largest group the bf16 backward takes
    # (the dK/dV kernels tag staged tiles with the head index 0 .. 31)
    "w2-gqa32": dict(wid=2, n=1024, h_q=32, h_kv=1, v_budget=100, s_budget=256),
    # 8 Q heads x 64 block-diagonals: early key blocks are read by up to 512
    # (head, query block) tiles, so the slash dK/dV kernel empties its tile list
    # and keeps appending (checked below by slash_tile_flushes).  Batch rows 1-15
    # carry empty lists: with 16 x 128 key blocks the launch has two rounds of
    # resident workgroups, so every key block's heads stay in one workgroup
    # (smaller grids split them over several) and its list holds all of them.
    "w2-flush-gqa8": dict(wid=2, n=8192, h_q=8, h_kv=1, v_budget=300, s_budget=4096, pad_batch=16),
}

# The slash dK/dV kernel collects the (head, query block) tiles of a key block
# in a list of KV_TILES entries, appending one head's selected block-diagonals
# KV_CHUNK at a time, and walks and empties the list whenever it holds more
# than KV_TILES - KV_CHUNK entries.
KV_TILES, KV_CHUNK = 512, 128


def slash_tile_flushes(index, h_q, h_kv, nb):
    """(max tiles of a key block, key blocks whose list is emptied with tiles after it)."""
    g_sz = h_q // h_kv
    most, after = 0, 0
    for grp in range(h_kv):
        diags = [np.asarray(index[(h, 0)][1]) for h in range(grp * g_sz, (grp + 1) * g_sz)]
        for j in range(nb):
            per_head = [int(((g > 0) & (j + g < nb)).sum()) for g in diags]
            most = max(most, sum(per_head))
            count, flushed, later = 0, False, 0
            for c in per_head:
                for base in range(0, c, KV_CHUNK):
                    count += min(KV_CHUNK, c - base)
                    if flushed:
                        later += min(KV_CHUNK, c - base)
                    if count > KV_TILES - KV_CHUNK:
                        count, flushed = 0, True
            after += int(flushed and later > 0)
    return most, after


def run_case(name, dev, check_index=True):
    kw = dict(CASES[name])
    pad_batch = kw.pop("pad_batch", 1)
    prob = workloads.make_problem(kw.pop("wid"), **kw)
    log(f"case {name}: n={prob.n} hq={prob.h_q} hkv={prob.h_kv} d={prob.d} dtype={prob.dtype} "
        f"docs={len(prob.cu_seqlens) - 1}")
    n_seg = len(prob.cu_seqlens) - 1
    oidx, oscores = oracle_index(prob)
    pos = np.arange(prob.n)
    q, k, v, do = (np64(t[0]) for t in (prob.q, prob.k, prob.v, prob.do))
    if prob.n <= 4096:
        O, L = oracle.attn_fwd_dense(q, k, v, pos, pos, prob.cu_seqlens, oidx)
    else:
        O, L = oracle.attn_fwd_support(q, k, v, pos, pos, prob.cu_seqlens, oidx)
    D = oracle.bwd_delta(O, do)
    if prob.n <= 4096:
        dq, dk, dv = oracle.attn_bwd_dense(q, k, v, do, L, D, pos, pos, prob.cu_seqlens, oidx)
    else:
        dq, dk, dv = oracle.attn_bwd_support(q, k, v, do, L, D, pos, pos, prob.cu_seqlens, oidx)

    if name == "w2-flush-gqa8":
        most, after = slash_tile_flushes(oidx, prob.h_q, prob.h_kv, prob.n // 64)
        log(f"  slash dK/dV tile lists: at most {most} tiles per key block, "
            f"{after} key blocks with tiles after the list was emptied")
        assert most > KV_TILES - KV_CHUNK and after > 0
    gq, gk, gv, gdo = (t.to(dev) for t in (prob.q, prob.k, prob.v, prob.do))
    cu = prob.cu_seqlens
    if check_index:
        gidx, vsc, ssc = vs.estimate_index(gq, gk, prob.v_budget, prob.s_budget, cu, return_scores=True)
        torch.cuda.synchronize()
        index_parity(name, oidx, oscores, [(a.numpy(), b.numpy()) for a, b in gidx.lists()],
                     vsc[0].cpu().numpy(), ssc[0].cpu().numpy(), prob)
    lists = lists_for_gpu(oidx, prob.h_q, n_seg)
    if pad_batch > 1:
        # batch rows 1.. : other inputs, no selected entries
        g = torch.Generator().manual_seed(prob.seed + 7)
        pad = [torch.randn((pad_batch - 1,) + tuple(t.shape[1:]), generator=g).to(t.dtype)
               for t in (prob.q, prob.k, prob.v, prob.do)]
        gq, gk, gv, gdo = (torch.cat([t, x]).to(dev) for t, x in zip((prob.q, prob.k, prob.v, prob.do), pad))
        lists = lists + [([], [])] * (len(lists) * (pad_batch - 1))
        log(f"  {pad_batch} batch rows, rows 1-{pad_batch - 1} with empty lists")
    idx = vs.index_from_lists(lists, dev)
    o, lse = vs.sparse_attn_fwd(gq, gk, gv, idx, cu)
    gdq, gdk, gdv = vs.sparse_attn_bwd(gq, gk, gv, o, gdo, lse, idx, cu_seqlens=cu)
    torch.cuda.synchronize()
    if pad_batch > 1:
        assert torch.isneginf(lse[1:]).all()
        for t in (o, gdq, gdk, gdv):
            assert not t[1:].float().abs().max().item(), "rows without selected entries must stay zero"
    bq = bk = bv = None
    if prob.dtype == "bf16":
        bq, bk, bv = oracle.bwd_rounding_bounds(q, k, v, do, O, L, pos, pos, prob.cu_seqlens, oidx)
    errs = [check_close(f"{name} O", O, np64(o[0]), prob.dtype, "o"),
            check_close(f"{name} LSE", L, lse[0].cpu().numpy().astype(np.float64), prob.dtype),
            check_close(f"{name} dQ", dq, np64(gdq[0]), prob.dtype, "grad", bq),
            check_close(f"{name} dK", dk, np64(gdk[0]), prob.dtype, "grad", bk),
            check_close(f"{name} dV", dv, np64(gdv[0]), prob.dtype, "grad", bv)]
    errs = [e for e in errs if e]
    assert not errs, errs
    return prob


@pytest.mark.parametrize("name", list(CASES))
def test_parity_small(name):
    run_case(name, _dev())


def test_delta_and_merge_kernels():
    dev = _dev()
    g = torch.Generator().manual_seed(7)
    B, N, H, d = 1, 512, 4, 128
    o = torch.randn((B, N, H, d), generator=g)
    do = torch.randn((B, N, H, d), generator=g).to(torch.bfloat16)
    delta = vs.attn_bwd_delta(o.to(dev), do.to(dev))
    ref = oracle.bwd_delta(np64(o[0]), np64(do[0]))
    assert_close("delta", ref, delta[0].cpu().numpy(), "f32")
    o1, o2 = torch.randn((2, B, N, H, d), generator=g)
    l1, l2 = torch.randn((2, B, H, N), generator=g) * 3
    l1[0, 0, :7] = -float("inf")
    l2[0, 0, 3:11] = -float("inf")
    o1[0, :7, 0] = 0
    o2[0, 3:11, 0] = 0
    acc_o, acc_l = o1.to(dev), l1.to(dev)
    vs.lse_merge(acc_o, acc_l, o2.to(dev), l2.to(dev))
    ro, rl = oracle.lse_merge(np64(o1[0]).transpose(1, 0, 2), np64(l1[0]), np64(o2[0]).transpose(1, 0, 2),
                              np64(l2[0]))
    assert_close("merge O", ro.transpose(1, 0, 2), acc_o[0].cpu().numpy(), "f32")
    assert_close("merge LSE", rl, acc_l[0].cpu().numpy(), "f32")


def test_striped_ring_share():
    """One worker's striped ring share: chunk calls + lse_merge = global rows (W=8),
    and the same with the merge fused into each chunk's forward."""
    dev = _dev()
    W, w = 8, 3
    prob = workloads.make_problem(4, n=8192, v_budget=512, s_budget=1536, stripe_world=W)
    oidx, _ = oracle_index(prob)
    q, k, v, do = (np64(t[0]) for t in (prob.q, prob.k, prob.v, prob.do))
    rows = workloads.stripe_positions(prob.n, W, w).numpy()
    pos = np.arange(prob.n)
    Og, Lg = oracle.attn_fwd_support(q, k, v, pos, pos, prob.cu_seqlens, oidx)
    Dg = oracle.bwd_delta(Og, do)
    dqg, dkg, dvg = oracle.attn_bwd_support(q, k, v, do, Lg, Dg, pos, pos, prob.cu_seqlens, oidx)
    idx = vs.index_from_lists(lists_for_gpu(oidx, prob.h_q, 1), dev)
    gq = workloads.stripe_rows(prob.q, W, w).to(dev)
    gdo = workloads.stripe_rows(prob.do, W, w).to(dev)
    nq = gq.shape[1]
    acc_o = torch.zeros((1, nq, prob.h_q, prob.d), device=dev)
    acc_l = torch.full((1, prob.h_q, nq), -float("inf"), device=dev)
    # the same ring share with the merge fused into the forward (o_f32 = 2)
    fused_o = torch.zeros_like(acc_o)
    fused_l = torch.full_like(acc_l, -float("inf"))
    chunks = []
    for t in range(W):
        u = (w - t) % W
        gk = workloads.stripe_rows(prob.k, W, u).to(dev)
        gv = workloads.stripe_rows(prob.v, W, u).to(dev)
        chunks.append((u, gk, gv))
        o, l = vs.sparse_attn_fwd(gq, gk, gv, idx, stripe=(W, w, u), o_f32=True)
        if t == 1:
            cols = workloads.stripe_positions(prob.n, W, u).numpy()
            Oc, Lc = oracle.attn_fwd_support(q[rows], k[cols], v[cols], rows, cols, prob.cu_seqlens, oidx)
            torch.cuda.synchronize()
            assert_close("chunk O", Oc, o[0].cpu().numpy(), "bf16", "o")
            assert_close("chunk LSE", Lc, l[0].cpu().numpy().astype(np.float64), "bf16")
        vs.lse_merge(acc_o, acc_l, o, l)
        vs.sparse_attn_fwd(gq, gk, gv, idx, stripe=(W, w, u), out=fused_o, lse=fused_l, merge=True)
    torch.cuda.synchronize()
    assert_close("merged O", Og[rows], acc_o[0].cpu().numpy(), "bf16", "o")
    assert_close("merged LSE", Lg[:, rows], acc_l[0].cpu().numpy().astype(np.float64), "bf16")
    assert_close("fused-merge O", Og[rows], fused_o[0].cpu().numpy(), "bf16", "o")
    assert_close("fused-merge LSE", Lg[:, rows], fused_l[0].cpu().numpy().astype(np.float64), "bf16")
    # fused and separate merges do the same fp32 arithmetic up to one rounding
    assert torch.allclose(fused_o, acc_o, rtol=1e-5, atol=1e-6)
    assert torch.equal(torch.isinf(fused_l), torch.isinf(acc_l))
    fin = torch.isfinite(acc_l)
    assert torch.allclose(fused_l[fin], acc_l[fin], rtol=1e-6, atol=1e-5)
    delta = vs.attn_bwd_delta(acc_o, gdo)
    dq = torch.zeros((1, nq, prob.h_q, prob.d), device=dev)
    dk_all = np.zeros_like(dkg)
    dv_all = np.zeros_like(dvg)
    for u, gk, gv in chunks:
        _, dk, dv = vs.sparse_attn_bwd(gq, gk, gv, None, gdo, acc_l, idx, delta=delta, dq=dq,
                                       stripe=(W, w, u), accumulate=True)
        cols = workloads.stripe_positions(prob.n, W, u).numpy()
        torch.cuda.synchronize()
        dk_all[cols] += np64(dk[0])
        dv_all[cols] += np64(dv[0])
    # worker w's share of dK/dV: the oracle restricted to its rows
    _, dkw, dvw = oracle.attn_bwd_support(q[rows], k, v, do[rows], Lg[:, rows], Dg[:, rows], rows, pos,
                                          prob.cu_seqlens, oidx)
    bq, bk, bv = oracle.bwd_rounding_bounds(q[rows], k, v, do[rows], Og[rows], Lg[:, rows], rows, pos,
                                            prob.cu_seqlens, oidx, u_o=2.0 ** -24, support=True)
    errs = [check_close("ring dQ", dqg[rows], np64(dq[0]), "bf16", "grad", bq),
            check_close("ring dK", dkw, dk_all, "bf16", "grad", bk),
            check_close("ring dV", dvw, dv_all, "bf16", "grad", bv)]
    errs = [e for e in errs if e]
    assert not errs, errs


def _topp_count_int(scores_f32, p):
    """The top-p count in the kernel's integer arithmetic (the decision the
    device takes, recomputed exactly from the device's own fp32 scores):
    masses rint(s * 2^54), target ceil(rint(p * 2^24) * total / 2^24)."""
    pc = np.float32(p)
    pc = np.float32(min(pc, np.float32(1.0))) if pc > 0 else np.float32(0.0)
    t = int(np.rint(np.float64(pc) * 2.0 ** 24))
    m = np.rint(np.asarray(scores_f32, np.float32).astype(np.float64) * 2.0 ** 54).astype(np.uint64)
    total = int(m.sum(dtype=np.uint64))
    if t == 0 or total == 0:
        return 0
    need = -(-(t * total) // (1 << 24))
    order = np.lexsort((np.arange(m.size), -np.asarray(scores_f32, np.float64)))
    c = np.cumsum([int(x) for x in m[order]], dtype=object)
    return int(np.argmax(np.array([x >= need for x in c]))) + 1


TOPP_CASES = {
    # name: (make_problem kwargs, caps v, caps s)
    "w2-n4096": (dict(wid=2, n=4096), [4096] * 8 + [60] * 8, [4096] * 8 + [640] * 8),
    "w5-n8192-docs": (dict(wid=5, n=8192, n_docs=4), [8192] * 16, [8192] * 16),
}


@pytest.mark.gpu
@pytest.mark.parametrize("name", list(TOPP_CASES))
def test_topp_index(name):
    """Top-p budgets (Algorithm 1 topp): device counts equal the integer
    definition on the device's scores; each list is the top-k of those scores
    padded with -1; counts and sets match the fp64 oracle or differ only within
    the certified bound; and attention on the padded index matches the oracle."""
    dev = _dev()
    kw, vcap, scap = TOPP_CASES[name]
    kw = dict(kw)
    prob = workloads.make_problem(kw.pop("wid"), **kw)
    hq, n_seg = prob.h_q, len(prob.cu_seqlens) - 1
    grid = [0.0, 0.05, 0.3, 0.5, 0.7, 0.9, 0.99, 1.0]
    p_v = [grid[h % 8] for h in range(hq)]
    p_s = [grid[(3 * h + 1) % 8] for h in range(hq)]
    log(f"case topp {name}: n={prob.n} hq={hq} docs={n_seg}")
    q, k = np64(prob.q[0]), np64(prob.k[0])
    oidx, osc, ocnt = oracle.estimate_index_topp(q, k, prob.cu_seqlens, vcap, scap, p_v, p_s, prob.block,
                                                 64, return_scores=True)
    gq, gk = prob.q.to(dev), prob.k.to(dev)
    gidx, gcnt, vsc, ssc = vs.estimate_index_topp(gq, gk, vcap, scap, p_v, p_s, prob.cu_seqlens,
                                                  return_scores=True)
    torch.cuda.synchronize()
    gl = [(a.numpy(), b.numpy()) for a, b in gidx.lists()]
    gcnt = gcnt.cpu().numpy()
    vsc, ssc = vsc[0].cpu().numpy(), ssc[0].cpu().numpy()
    flips = swaps = 0
    for h in range(hq):
        for s in range(n_seg):
            a, e = prob.cu_seqlens[s], prob.cu_seqlens[s + 1]
            l = h * n_seg + s
            cv, cg = oracle.capacities(vcap[h], scap[h], e - a, prob.n, prob.block)
            for kind, pp, cap, gsc, osc_k, off in (
                    (0, p_v[h], cv, vsc[h, a:e], osc[(h, s)][0], a),
                    (1, p_s[h], cg, ssc[h, a // 64:e // 64], osc[(h, s)][1], 0)):
                kg = int(gcnt[l, kind])
                # 1. the device's decision, exactly
                assert kg == min(_topp_count_int(gsc, pp), cap), (name, h, s, kind, kg)
                # 2. the list: top-kg of the device's scores, ascending, then -1
                lst = gl[l][kind]
                assert lst.size == cap and np.all(lst[kg:] == -1), (name, h, s, kind)
                order = np.lexsort((np.arange(gsc.size), -np.asarray(gsc, np.float64)))
                assert np.array_equal(lst[:kg], np.sort(order[:kg]) + off), (name, h, s, kind)
                # 3. against the fp64 oracle
                ko = ocnt[(h, s)][kind]
                o64 = np.asarray(osc_k, np.float64)
                if kg != ko:
                    so = np.sort(o64)[::-1]
                    cum = np.concatenate(([0.0], np.cumsum(so)))
                    tot = cum[-1]
                    delta = 2 * np.abs(np.asarray(gsc, np.float64) - o64).sum() + 2.0 ** -24 * tot + 1e-12
                    pc = min(pp, 1.0)
                    # the device's uncapped count reaches the target at kg (unless
                    # capped) and not before it, up to the score differences
                    assert kg == cap or cum[kg] >= pc * tot - delta, (name, h, s, kind, kg, ko)
                    assert kg == 0 or cum[kg - 1] < pc * tot + delta, (name, h, s, kind, kg, ko)
                    flips += 1
                ref = oracle.select_topk(o64, kg) + off
                if not np.array_equal(np.sort(ref), lst[:kg]):
                    kth = np.sort(o64)[::-1][kg - 1]
                    extra = np.setdiff1d(lst[:kg], ref) - off
                    miss = np.setdiff1d(ref, lst[:kg]) - off
                    tol = 1e-4 * max(kth, 1e-30)
                    assert np.all(np.abs(o64[extra] - kth) <= tol) and np.all(np.abs(o64[miss] - kth) <= tol), \
                        (name, h, s, kind, "non-tie mismatch")
                    swaps += extra.size
    log(f"  topp {name}: counts match (certified boundary flips={flips}), near-tie swaps={swaps}")
    # attention on the padded device index against the oracle on the same lists
    lists = {(h, s): (gl[h * n_seg + s][0][gl[h * n_seg + s][0] >= 0].astype(np.int64),
                      gl[h * n_seg + s][1][gl[h * n_seg + s][1] >= 0].astype(np.int64))
             for h in range(hq) for s in range(n_seg)}
    v_, do_ = np64(prob.v[0]), np64(prob.do[0])
    pos = np.arange(prob.n)
    O, L = oracle.attn_fwd_support(q, k, v_, pos, pos, prob.cu_seqlens, lists)
    D = oracle.bwd_delta(O, do_)
    dq, dk, dv = oracle.attn_bwd_support(q, k, v_, do_, L, D, pos, pos, prob.cu_seqlens, lists)
    gv, gdo = prob.v.to(dev), prob.do.to(dev)
    o, lse = vs.sparse_attn_fwd(gq, gk, gv, gidx, prob.cu_seqlens)
    gdq, gdk, gdv = vs.sparse_attn_bwd(gq, gk, gv, o, gdo, lse, gidx, cu_seqlens=prob.cu_seqlens)
    torch.cuda.synchronize()
    bq, bk, bv = oracle.bwd_rounding_bounds(q, k, v_, do_, O, L, pos, pos, prob.cu_seqlens, lists)
    errs = [check_close(f"topp {name} O", O, np64(o[0]), prob.dtype, "o"),
            check_close(f"topp {name} LSE", L, lse[0].cpu().numpy().astype(np.float64), prob.dtype),
            check_close(f"topp {name} dQ", dq, np64(gdq[0]), prob.dtype, "grad", bq),
            check_close(f"topp {name} dK", dk, np64(gdk[0]), prob.dtype, "grad", bk),
            check_close(f"topp {name} dV", dv, np64(gdv[0]), prob.dtype, "grad", bv)]
    errs = [e for e in errs if e]
    assert not errs, errs


@pytest.mark.gpu
@pytest.mark.parametrize("wid,dtype,d", [(1, "f32", 64), (2, "bf16", 64)])
def test_fused_merge_other_kernels(wid, dtype, d):
    """The merge fused into the forward (o_f32 = 2) in the fp32 kernel and the
    d = 64 bf16 kernel: two striped KV chunks merged in the epilogue equal the
    same chunks merged by lse_merge, and the oracle's global rows."""
    dev = _dev()
    W, w = 2, 1
    prob = workloads.make_problem(wid, n=2048, h_q=2, h_kv=1, d=d, dtype=dtype, v_budget=150,
                                  s_budget=400, stripe_world=W)
    oidx, _ = oracle_index(prob)
    q, k, v = (np64(t[0]) for t in (prob.q, prob.k, prob.v))
    pos = np.arange(prob.n)
    Og, Lg = oracle.attn_fwd_support(q, k, v, pos, pos, prob.cu_seqlens, oidx)
    rows = workloads.stripe_positions(prob.n, W, w).numpy()
    idx = vs.index_from_lists(lists_for_gpu(oidx, prob.h_q, 1), dev)
    gq = workloads.stripe_rows(prob.q, W, w).to(dev)
    nq = gq.shape[1]
    sep_o = torch.zeros((1, nq, prob.h_q, prob.d), device=dev)
    sep_l = torch.full((1, prob.h_q, nq), -float("inf"), device=dev)
    fused_o, fused_l = torch.zeros_like(sep_o), torch.full_like(sep_l, -float("inf"))
    for u in range(W):
        gk = workloads.stripe_rows(prob.k, W, u).to(dev)
        gv = workloads.stripe_rows(prob.v, W, u).to(dev)
        o, l = vs.sparse_attn_fwd(gq, gk, gv, idx, stripe=(W, w, u), o_f32=True)
        vs.lse_merge(sep_o, sep_l, o, l)
        vs.sparse_attn_fwd(gq, gk, gv, idx, stripe=(W, w, u), out=fused_o, lse=fused_l, merge=True)
    torch.cuda.synchronize()
    assert torch.allclose(fused_o, sep_o, rtol=1e-5, atol=1e-6)
    fin = torch.isfinite(sep_l)
    assert torch.equal(fin, torch.isfinite(fused_l)) and torch.allclose(fused_l[fin], sep_l[fin], rtol=1e-6, atol=1e-5)
    assert_close("fused-merge O", Og[rows], fused_o[0].cpu().numpy(), prob.dtype, "o")
    assert_close("fused-merge LSE", Lg[:, rows], fused_l[0].cpu().numpy().astype(np.float64), prob.dtype)


def test_batch2():
    """Two different sequences in one call (batch = 2): estimator, forward and
    backward, each batch row against the oracle on its own inputs and index."""
    dev = _dev()
    kw = dict(n=2048, h_q=4, h_kv=2, v_budget=150, s_budget=500)
    probs = [workloads.make_problem(2, **kw), workloads.make_problem(2, seed=2017, **kw)]
    p0 = probs[0]
    cat = lambda name: torch.cat([getattr(p, name) for p in probs], dim=0)
    gq, gk, gv, gdo = (cat(n).to(dev) for n in ("q", "k", "v", "do"))
    log(f"case batch2: n={p0.n} hq={p0.h_q} hkv={p0.h_kv}")
    gidx, vsc, ssc = vs.estimate_index(gq, gk, p0.v_budget, p0.s_budget, return_scores=True)
    torch.cuda.synchronize()
    glists = [(a.numpy(), b.numpy()) for a, b in gidx.lists()]
    olists = []
    refs = []
    for b, prob in enumerate(probs):
        oidx, osc = oracle_index(prob)
        index_parity(f"batch2 row {b}", oidx, osc, glists[b * p0.h_q:(b + 1) * p0.h_q],
                     vsc[b].cpu().numpy(), ssc[b].cpu().numpy(), prob)
        olists += lists_for_gpu(oidx, prob.h_q, 1)
        q, k, v, do = (np64(t[0]) for t in (prob.q, prob.k, prob.v, prob.do))
        pos = np.arange(prob.n)
        O, L = oracle.attn_fwd_dense(q, k, v, pos, pos, prob.cu_seqlens, oidx)
        D = oracle.bwd_delta(O, do)
        grads = oracle.attn_bwd_dense(q, k, v, do, L, D, pos, pos, prob.cu_seqlens, oidx)
        bounds = oracle.bwd_rounding_bounds(q, k, v, do, O, L, pos, pos, prob.cu_seqlens, oidx)
        refs.append((O, L, grads, bounds))
    idx = vs.index_from_lists(olists, dev)
    o, lse = vs.sparse_attn_fwd(gq, gk, gv, idx)
    gdq, gdk, gdv = vs.sparse_attn_bwd(gq, gk, gv, o, gdo, lse, idx)
    torch.cuda.synchronize()
    errs = []
    for b, (O, L, (dq, dk, dv), (bq, bk, bv)) in enumerate(refs):
        errs += [check_close(f"batch2 row {b} O", O, np64(o[b]), "bf16", "o"),
                 check_close(f"batch2 row {b} LSE", L, lse[b].cpu().numpy().astype(np.float64), "bf16"),
                 check_close(f"batch2 row {b} dQ", dq, np64(gdq[b]), "bf16", "grad", bq),
                 check_close(f"batch2 row {b} dK", dk, np64(gdk[b]), "bf16", "grad", bk),
                 check_close(f"batch2 row {b} dV", dv, np64(gdv[b]), "bf16", "grad", bv)]
    errs = [e for e in errs if e]
    assert not errs, errs


def _tie_problem():
    """Inputs with exact score ties for the estimator (no rounding decides them).

    KV group 1 (Q heads 2, 3): the observation-window rows of Q are zero, so
    every score there is 0: every column before the window gets the same
    vertical score and every full block-diagonal the same slash score.
    KV group 0 (Q heads 0, 1): 40 key rows before the window are one and the
    same row 20 u (u a unit vector), and every window query of heads 0, 1 has
    component 2 along u, so those 40 columns score 40 / sqrt(d) (about 3.5)
    in every window row, above the other keys (no outlier keys are drawn), and
    share the largest vertical score; the budget keeps 24 of them.  The tie
    rule (lowest index first) alone decides which.  (A larger score would put
    nearly all of a row's probability on the copies, where dQ becomes a sum of
    large dS terms that cancel, beyond what bf16 products can resolve.)
    """
    prob = workloads.make_problem(2, n=2048, h_q=4, h_kv=2, v_budget=[24, 24, 100, 100],
                                  s_budget=[448, 448, 640, 640], out_frac=0.0)
    n = prob.n
    q, k = prob.q.to(torch.float32), prob.k.clone()
    q[0, n - 64:, 2:4] = 0
    g = torch.Generator().manual_seed(99)
    u = torch.randn(prob.d, generator=g)
    u = u / u.norm()
    w = q[0, n - 64:, 0:2]
    q[0, n - 64:, 0:2] = w - (w @ u)[..., None] * u + 2.0 * u
    copies = torch.arange(37, 37 + 40 * 43, 43)
    assert int(copies[-1]) < n - 64
    k[0, copies, 0] = (20.0 * u).to(k.dtype)
    prob.q, prob.k = q.to(prob.q.dtype), k
    return prob, copies


def test_tie_index():
    """Exact ties in the estimator's scores are broken by the lowest index on
    the GPU as in the oracle: the lists must be equal, with no near-tie
    allowance; attention on that index matches the oracle."""
    dev = _dev()
    prob, copies = _tie_problem()
    oidx, osc = oracle_index(prob)
    # the fixture does what it claims: the oracle's lists are the lowest-index
    # members of the tied sets
    for h in (0, 1):
        assert np.array_equal(oidx[(h, 0)][0], copies[:24].numpy()), h
    nb = prob.n // 64
    for h in (2, 3):
        assert np.array_equal(oidx[(h, 0)][0], np.arange(100)), h
        assert np.array_equal(oidx[(h, 0)][1], np.arange(1, 11)), h
        assert np.ptp(osc[(h, 0)][1][1:]) == 0 and osc[(h, 0)][1][0] < osc[(h, 0)][1][1]
    gq, gk, gv, gdo = (t.to(dev) for t in (prob.q, prob.k, prob.v, prob.do))
    gidx, vsc, ssc = vs.estimate_index(gq, gk, prob.v_budget, prob.s_budget, return_scores=True)
    torch.cuda.synchronize()
    glists = [(a.numpy(), b.numpy()) for a, b in gidx.lists()]
    vsc, ssc = vsc[0].cpu().numpy(), ssc[0].cpu().numpy()
    for h in range(prob.h_q):
        # the device's own scores tie exactly where the inputs make them tie
        tied = copies.numpy() if h < 2 else np.arange(prob.n - 64)
        assert np.ptp(vsc[h, tied]) == 0, (h, "vertical scores of tied columns differ")
        assert np.array_equal(glists[h][0], oidx[(h, 0)][0]), (h, glists[h][0][:30])
        if h >= 2:
            assert np.ptp(ssc[h, 1:nb]) == 0, (h, "slash scores of full block-diagonals differ")
            assert np.array_equal(glists[h][1], oidx[(h, 0)][1]), (h, glists[h][1])
    # heads 0, 1: their block-diagonal scores differ only by terms far below
    # fp32 resolution, so those lists follow the usual certified comparison
    index_parity("tie case", oidx, osc, glists, vsc, ssc, prob)
    log("  tie case: GPU lists equal the oracle's exactly (lowest index among exact ties)")
    idx = vs.index_from_lists(lists_for_gpu(oidx, prob.h_q, 1), dev)
    q, k, v, do = (np64(t[0]) for t in (prob.q, prob.k, prob.v, prob.do))
    pos = np.arange(prob.n)
    O, L = oracle.attn_fwd_dense(q, k, v, pos, pos, prob.cu_seqlens, oidx)
    D = oracle.bwd_delta(O, do)
    dq, dk, dv = oracle.attn_bwd_dense(q, k, v, do, L, D, pos, pos, prob.cu_seqlens, oidx)
    bq, bk, bv = oracle.bwd_rounding_bounds(q, k, v, do, O, L, pos, pos, prob.cu_seqlens, oidx)
    o, lse = vs.sparse_attn_fwd(gq, gk, gv, idx)
    gdq, gdk, gdv = vs.sparse_attn_bwd(gq, gk, gv, o, gdo, lse, idx)
    torch.cuda.synchronize()
    errs = [check_close("tie O", O, np64(o[0]), "bf16", "o"),
            check_close("tie LSE", L, lse[0].cpu().numpy().astype(np.float64), "bf16"),
            check_close("tie dQ", dq, np64(gdq[0]), "bf16", "grad", bq),
            check_close("tie dK", dk, np64(gdk[0]), "bf16", "grad", bk),
            check_close("tie dV", dv, np64(gdv[0]), "bf16", "grad", bv)]
    errs = [e for e in errs if e]
    assert not errs, errs


def test_topp_long_lists_two_stage():
    """Top-p counts on lists of 32768 columns (N = 32768), where the top-k
    runs in two stages (per-chunk selections, then their merge) with the
    device's counts: every count is the integer top-p decision on the
    device's own scores, and every list is the top-count of those scores
    (ties to the lowest index), ascending, padded with -1."""
    dev = _dev()
    prob = workloads.make_problem(2, n=32768, h_q=8, h_kv=2)
    hq = prob.h_q
    grid = [0.05, 0.3, 0.5, 0.7, 0.9, 0.95, 0.99, 1.0]
    p_v = [grid[h % 8] for h in range(hq)]
    p_s = [grid[(3 * h + 1) % 8] for h in range(hq)]
    vcap, scap = [8192] * hq, [32768] * hq
    gidx, gcnt, vsc, ssc = vs.estimate_index_topp(prob.q.to(dev), prob.k.to(dev), vcap, scap, p_v, p_s,
                                                  prob.cu_seqlens, return_scores=True)
    torch.cuda.synchronize()
    gl = [(a.numpy(), b.numpy()) for a, b in gidx.lists()]
    gcnt = gcnt.cpu().numpy()
    vsc, ssc = vsc[0].cpu().numpy(), ssc[0].cpu().numpy()
    two_stage = 0
    for h in range(hq):
        cv, cg = oracle.capacities(vcap[h], scap[h], prob.n, prob.n, prob.block)
        for kind, pp, cap, gsc in ((0, p_v[h], cv, vsc[h]), (1, p_s[h], cg, ssc[h])):
            kg = int(gcnt[h, kind])
            assert kg == min(_topp_count_int(gsc, pp), cap), (h, kind, kg)
            lst = gl[h][kind]
            assert lst.size == cap and np.all(lst[kg:] == -1), (h, kind)
            order = np.lexsort((np.arange(gsc.size), -np.asarray(gsc, np.float64)))
            assert np.array_equal(lst[:kg], np.sort(order[:kg])), (h, kind)
            two_stage += kind == 0 and 0 < kg < gsc.size and 2 * kg <= 16384
    assert two_stage >= 4, two_stage  # the case exercises the two-stage select
    log(f"  topp on 32768-column lists: counts and lists exact ({two_stage} two-stage lists)")


def test_topk_ties_beyond_gathered_bin():
    """The top-k select gathers the entries of the k-th score's leading 11-bit
    bin in LDS (up to 8192); here the observation-window rows of Q are zero,
    so the 16320 columns before the window share one vertical score: the
    select takes its radix passes over the whole list instead, and the lists
    still equal the oracle's (the lowest indices among the ties)."""
    dev = _dev()
    prob = workloads.make_problem(2, n=16384, h_q=2, h_kv=1, v_budget=[100, 100], s_budget=[640, 640],
                                  out_frac=0.0)
    n = prob.n
    q = prob.q.to(torch.float32)
    q[0, n - 64:] = 0
    prob.q = q.to(prob.q.dtype)
    oidx, _ = oracle_index(prob)
    for h in range(2):
        assert np.array_equal(oidx[(h, 0)][0], np.arange(100)), h
    gidx, vsc, _ = vs.estimate_index(prob.q.to(dev), prob.k.to(dev), prob.v_budget, prob.s_budget,
                                     return_scores=True)
    torch.cuda.synchronize()
    vsc = vsc[0].cpu().numpy()
    glists = [(a.numpy(), b.numpy()) for a, b in gidx.lists()]
    for h in range(2):
        assert np.ptp(vsc[h, :n - 64]) == 0, (h, "tied vertical scores differ")
        assert np.array_equal(glists[h][0], oidx[(h, 0)][0]), (h, glists[h][0][:20])
        assert np.array_equal(glists[h][1], oidx[(h, 0)][1]), (h, glists[h][1])
    log("  top-k with 16320 tied scores: lists equal the oracle's")


@pytest.mark.parametrize("dtype,d,h_q,h_kv", [("bf16", 128, 4, 2), ("f32", 64, 2, 1)])
def test_fused_qkv_strides(dtype, d, h_q, h_kv):
    """Q, K, V as slices of one fused [batch, token, h_q + 2 h_kv, d] projection
    (token stride (h_q + 2 h_kv) d), dO and O as views with padded heads, batch
    2: estimator, forward and backward through the strides, against the oracle
    on each batch row."""
    dev = _dev()
    kw = dict(n=2048, h_q=h_q, h_kv=h_kv, d=d, dtype=dtype, v_budget=150, s_budget=500)
    probs = [workloads.make_problem(2, **kw), workloads.make_problem(2, seed=2027, **kw)]
    p0 = probs[0]
    B, N, td = len(probs), p0.n, p0.torch_dtype
    qkv = torch.empty((B, N, h_q + 2 * h_kv, d), dtype=td, device=dev)
    do_buf = torch.zeros((B, N, h_q, 2 * d), dtype=td, device=dev)
    o_buf = torch.zeros((B, N, h_q, d + 64), dtype=td, device=dev)
    for b, pr in enumerate(probs):
        qkv[b, :, :h_q] = pr.q[0].to(dev)
        qkv[b, :, h_q:h_q + h_kv] = pr.k[0].to(dev)
        qkv[b, :, h_q + h_kv:] = pr.v[0].to(dev)
        do_buf[b, :, :, :d] = pr.do[0].to(dev)
    q, k, v = qkv[:, :, :h_q], qkv[:, :, h_q:h_q + h_kv], qkv[:, :, h_q + h_kv:]
    do, o = do_buf[..., :d], o_buf[..., :d]
    assert q.stride(1) == (h_q + 2 * h_kv) * d and not q.is_contiguous() and not o.is_contiguous()
    log(f"case fused-qkv {dtype}: batch {B}, n={N}, token stride {q.stride(1)}")
    gidx, vsc, ssc = vs.estimate_index(q, k, p0.v_budget, p0.s_budget, return_scores=True)
    torch.cuda.synchronize()
    glists = [(a.numpy(), b.numpy()) for a, b in gidx.lists()]
    olists, refs = [], []
    for b, prob in enumerate(probs):
        oidx, osc = oracle_index(prob)
        index_parity(f"fused-qkv row {b}", oidx, osc, glists[b * h_q:(b + 1) * h_q],
                     vsc[b].cpu().numpy(), ssc[b].cpu().numpy(), prob)
        olists += lists_for_gpu(oidx, h_q, 1)
        qq, kk, vv, dd = (np64(t[0]) for t in (prob.q, prob.k, prob.v, prob.do))
        pos = np.arange(N)
        O, L = oracle.attn_fwd_dense(qq, kk, vv, pos, pos, prob.cu_seqlens, oidx)
        D = oracle.bwd_delta(O, dd)
        grads = oracle.attn_bwd_dense(qq, kk, vv, dd, L, D, pos, pos, prob.cu_seqlens, oidx)
        bounds = (oracle.bwd_rounding_bounds(qq, kk, vv, dd, O, L, pos, pos, prob.cu_seqlens, oidx)
                  if dtype == "bf16" else (None, None, None))
        refs.append((O, L, grads, bounds))
    idx = vs.index_from_lists(olists, dev)
    _, lse = vs.sparse_attn_fwd(q, k, v, idx, out=o)
    gdq, gdk, gdv = vs.sparse_attn_bwd(q, k, v, o, do, lse, idx)
    torch.cuda.synchronize()
    assert float(o_buf[..., d:].abs().max()) == 0.0, "writes outside the O view"
    errs = []
    for b, (O, L, (dq, dk, dv), (bq, bk, bv)) in enumerate(refs):
        errs += [check_close(f"fused-qkv row {b} O", O, np64(o[b]), dtype, "o"),
                 check_close(f"fused-qkv row {b} LSE", L, lse[b].cpu().numpy().astype(np.float64), dtype),
                 check_close(f"fused-qkv row {b} dQ", dq, np64(gdq[b]), dtype, "grad", bq),
                 check_close(f"fused-qkv row {b} dK", dk, np64(gdk[b]), dtype, "grad", bk),
                 check_close(f"fused-qkv row {b} dV", dv, np64(gdv[b]), dtype, "grad", bv)]
    errs = [e for e in errs if e]
    assert not errs, errs


def test_all_chunks_one_call():
    """A striped worker's whole ring in one call (k_rank = all chunks, W = 8):
    K / V hold the 8 chunks one after the other; O, LSE and dQ equal the
    oracle's global rows, dK / dV of every chunk the worker's share of the
    global gradients; and the result agrees with the 8-step ring of chunk
    calls (merge fused, dQ accumulated)."""
    dev = _dev()
    W, w = 8, 5
    prob = workloads.make_problem(4, n=8192, v_budget=512, s_budget=1536, stripe_world=W)
    oidx, _ = oracle_index(prob)
    q, k, v, do = (np64(t[0]) for t in (prob.q, prob.k, prob.v, prob.do))
    rows = workloads.stripe_positions(prob.n, W, w).numpy()
    pos = np.arange(prob.n)
    Og, Lg = oracle.attn_fwd_support(q, k, v, pos, pos, prob.cu_seqlens, oidx)
    Dg = oracle.bwd_delta(Og, do)
    _, dkw, dvw = oracle.attn_bwd_support(q[rows], k, v, do[rows], Lg[:, rows], Dg[:, rows], rows, pos,
                                          prob.cu_seqlens, oidx)
    dqg, _, _ = oracle.attn_bwd_support(q, k, v, do, Lg, Dg, pos, pos, prob.cu_seqlens, oidx)
    idx = vs.index_from_lists(lists_for_gpu(oidx, prob.h_q, 1), dev)
    gq = workloads.stripe_rows(prob.q, W, w).to(dev)
    gdo = workloads.stripe_rows(prob.do, W, w).to(dev)
    chunk_pos = np.concatenate([workloads.stripe_positions(prob.n, W, u).numpy() for u in range(W)])
    cp = torch.from_numpy(chunk_pos)
    k_all = prob.k[:, cp].contiguous().to(dev)
    v_all = prob.v[:, cp].contiguous().to(dev)
    log(f"case all-chunks: n={prob.n} W={W} worker {w}")
    o, lse = vs.sparse_attn_fwd(gq, k_all, v_all, idx, stripe=(W, w, "all"))
    o32, lse32 = vs.sparse_attn_fwd(gq, k_all, v_all, idx, stripe=(W, w, "all"), o_f32=True)
    dq, dk, dv = vs.sparse_attn_bwd(gq, k_all, v_all, o, gdo, lse, idx, stripe=(W, w, "all"))
    # the same worker's ring of W chunk calls
    nq = gq.shape[1]
    acc_o = torch.zeros((1, nq, prob.h_q, prob.d), device=dev)
    acc_l = torch.full((1, prob.h_q, nq), -float("inf"), device=dev)
    chunks = []
    for t in range(W):
        u = (w - t) % W
        chunks.append((u, workloads.stripe_rows(prob.k, W, u).to(dev), workloads.stripe_rows(prob.v, W, u).to(dev)))
    for u, gk, gv in chunks:
        vs.sparse_attn_fwd(gq, gk, gv, idx, stripe=(W, w, u), out=acc_o, lse=acc_l, merge=True)
    torch.cuda.synchronize()
    bq, bk, bv = oracle.bwd_rounding_bounds(q[rows], k, v, do[rows], Og[rows], Lg[:, rows], rows, pos,
                                            prob.cu_seqlens, oidx, support=True)
    dk_g = np.zeros_like(dkw)
    dv_g = np.zeros_like(dvw)
    dk_g[chunk_pos] = np64(dk[0])
    dv_g[chunk_pos] = np64(dv[0])
    errs = [check_close("all-chunks O", Og[rows], np64(o[0]), "bf16", "o"),
            check_close("all-chunks LSE", Lg[:, rows], lse[0].cpu().numpy().astype(np.float64), "bf16"),
            check_close("all-chunks O (fp32 out)", Og[rows], np64(o32[0]), "bf16", "o"),
            check_close("all-chunks dQ", dqg[rows], np64(dq[0]), "bf16", "grad", bq),
            check_close("all-chunks dK", dkw, dk_g, "bf16", "grad", bk),
            check_close("all-chunks dV", dvw, dv_g, "bf16", "grad", bv)]
    errs = [e for e in errs if e]
    assert not errs, errs
    # one call and the ring compute the same rows; the probabilities are
    # rounded to bf16 against different running maxima (all chunks at once vs
    # one chunk at a time), so O agrees to the bf16 tolerance and LSE (fp32
    # sums) closely
    err = float((o32 - acc_o).abs().max())
    log(f"  all-chunks vs ring: O max-abs {err:.3e}")
    assert err <= 2e-2
    fin = torch.isfinite(acc_l)
    assert torch.equal(fin, torch.isfinite(lse32)) and torch.allclose(lse32[fin], acc_l[fin], rtol=1e-5, atol=1e-4)
