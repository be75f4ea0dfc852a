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
}


def run_case(name, dev, check_index=True):
    kw = dict(CASES[name])
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

    gq, gk, gv, gdo = (t.to(dev) for t in (prob.q, prob.k, prob.v, prob.do))
    cu = prob.cu_seqlens
    if check_index:
        gidx, vsc, ssc = vs.estimate_index(gq, gk, prob.v_budget, prob.s_budget, cu, return_scores=True)
        torch.cuda.synchronize()
        index_parity(name, oidx, oscores, [(a.numpy(), b.numpy()) for a, b in gidx.lists()],
                     vsc[0].cpu().numpy(), ssc[0].cpu().numpy(), prob)
    idx = vs.index_from_lists(lists_for_gpu(oidx, prob.h_q, n_seg), dev)
    o, lse = vs.sparse_attn_fwd(gq, gk, gv, idx, cu)
    gdq, gdk, gdv = vs.sparse_attn_bwd(gq, gk, gv, o, gdo, lse, idx, cu_seqlens=cu)
    torch.cuda.synchronize()
    bq = bk = bv = None
    if prob.dtype == "bf16":
        bq, bk, bv = oracle.bwd_rounding_bounds(q, k, v, do, O, L, pos, pos, prob.cu_seqlens, oidx)
    errs = [check_close(f"{name} O", O, np64(o[0]), prob.dtype),
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
    """One worker's striped ring share: chunk calls + lse_merge = global rows (W=8)."""
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
            assert_close("chunk O", Oc, o[0].cpu().numpy(), "bf16")
            assert_close("chunk LSE", Lc, l[0].cpu().numpy().astype(np.float64), "bf16")
        vs.lse_merge(acc_o, acc_l, o, l)
    torch.cuda.synchronize()
    assert_close("merged O", Og[rows], acc_o[0].cpu().numpy(), "bf16")
    assert_close("merged LSE", Lg[:, rows], acc_l[0].cpu().numpy().astype(np.float64), "bf16")
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
