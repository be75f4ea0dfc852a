"""A striped worker's ring captured as a HIP graph and replayed (GPU).

The ring of one worker (W = 8 ranks, 64-token stripes, N = 8192): a forward
call per KV chunk merging into the running (O, LSE), delta, and a backward call
per chunk accumulating dQ, each chunk's dK / dV in its own buffer.  Captured
once, the graph is replayed three times; before each replay the same ring runs
eagerly into other buffers and the stream is synchronised, and every replay's
results must equal the eager ones (O, LSE and dQ bit for bit; dK and dV, which
take fp32 atomics in an order that may differ from run to run, within 1e-5 of
their largest value).  The eager ring's O is checked against the oracle's
global rows.
"""
import numpy as np
import pytest
import torch

import dynamic_sparse_attention_amd as vs
import oracle
import workloads
from vs_cases import assert_close, lists_for_gpu, log, np64, oracle_index

pytestmark = pytest.mark.gpu


def test_ring_graph_replays_match_eager():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dev = torch.device("cuda:0")
    W, w = 8, 3
    prob = workloads.make_problem(4, n=8192, v_budget=512, s_budget=1536, stripe_world=W)
    log(f"case ring graph: n={prob.n} W={W} worker={w} hq={prob.h_q} hkv={prob.h_kv}")
    oidx, _ = oracle_index(prob)
    idx = vs.index_from_lists(lists_for_gpu(oidx, prob.h_q, 1), dev)
    gq = workloads.stripe_rows(prob.q, W, w).to(dev)
    gdo = workloads.stripe_rows(prob.do, W, w).to(dev)
    nq = gq.shape[1]
    chunks = []
    for t in range(W):
        u = (w - t) % W
        chunks.append((u, workloads.stripe_rows(prob.k, W, u).to(dev), workloads.stripe_rows(prob.v, W, u).to(dev)))

    def buffers():
        return dict(o=torch.empty((1, nq, prob.h_q, prob.d), device=dev),
                    l=torch.empty((1, prob.h_q, nq), device=dev),
                    dq=torch.empty((1, nq, prob.h_q, prob.d), device=dev),
                    kv=[(torch.empty((1, nq, prob.h_kv, prob.d), device=dev),
                         torch.empty((1, nq, prob.h_kv, prob.d), device=dev)) for _ in range(W)])

    def ring(b):
        b["o"].zero_()
        b["l"].fill_(-float("inf"))
        for u, gk, gv in chunks:
            vs.sparse_attn_fwd(gq, gk, gv, idx, stripe=(W, w, u), out=b["o"], lse=b["l"], merge=True)
        delta = vs.attn_bwd_delta(b["o"], gdo)
        b["dq"].zero_()
        for (u, gk, gv), (dk, dv) in zip(chunks, b["kv"]):
            vs.sparse_attn_bwd(gq, gk, gv, None, gdo, b["l"], idx, delta=delta, dq=b["dq"], dk=dk, dv=dv,
                               stripe=(W, w, u), accumulate=True)

    eager, replayed = buffers(), buffers()
    ring(eager)  # first calls outside the capture (workspace, lazy set-up)
    ring(replayed)
    torch.cuda.synchronize()
    q, k, v = (np64(t[0]) for t in (prob.q, prob.k, prob.v))
    rows = workloads.stripe_positions(prob.n, W, w).numpy()
    pos = np.arange(prob.n)
    Og, Lg = oracle.attn_fwd_support(q, k, v, pos, pos, prob.cu_seqlens, oidx)
    assert_close("eager ring O", Og[rows], eager["o"][0].cpu().numpy(), "bf16", "o")

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ring(replayed)
    for r in range(3):
        for t in (eager["o"], eager["dq"]):
            t.fill_(float("nan"))  # the eager ring must write them again
        ring(eager)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        log(f"  replay {r}")
        assert torch.equal(replayed["o"], eager["o"]), r
        assert torch.equal(replayed["l"], eager["l"]), r
        assert torch.equal(replayed["dq"], eager["dq"]), r
        worst = 0.0
        for u, ((a, b), (c, e)) in enumerate(zip(replayed["kv"], eager["kv"])):
            for name, x, y in (("dK", a, c), ("dV", b, e)):
                # fp32 atomics add in an order that may differ between runs:
                # differences at the rounding of the array's largest values
                err = float((x - y).abs().max())
                scale = float(y.abs().max())
                worst = max(worst, err / max(scale, 1.0))
                assert err <= 1e-5 * max(scale, 1.0), (r, u, name, err, scale)
        log(f"    dK / dV: largest difference {worst:.2e} of max(|eager|, 1)")
