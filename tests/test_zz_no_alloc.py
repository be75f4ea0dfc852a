"""The allocation-free backward entry point (vs_sparse_attn_bwd_noalloc)
against vs_sparse_attn_bwd, through the C ABI, on two calls in a row (the
second on a smaller problem of the other dtype), so that the shared scratch
array carries the first call's contents into the second."""
import numpy as np
import pytest
import torch

import workloads
from vs_cases import log

pytestmark = pytest.mark.gpu

vs = pytest.importorskip("dynamic_sparse_attention_amd")


def _one_call(dev, wid, **kw):
    prob = workloads.make_problem(wid, **kw)
    q, k, v, do = (t.to(dev) for t in (prob.q, prob.k, prob.v, prob.do))
    idx = vs.estimate_index(q, k, prob.v_budget, prob.s_budget, prob.cu_seqlens)
    o, lse = vs.sparse_attn_fwd(q, k, v, idx, prob.cu_seqlens)
    ref = vs.sparse_attn_bwd(q, k, v, o, do, lse, idx, cu_seqlens=prob.cu_seqlens)
    got = vs.sparse_attn_bwd_noalloc(q, k, v, o, do, lse, idx, cu_seqlens=prob.cu_seqlens)
    torch.cuda.synchronize()
    log(f"noalloc {prob.dtype} n={prob.n} hq={prob.h_q} hkv={prob.h_kv} d={prob.d}")
    # same kernels on the same inputs: dQ (no atomics) is bit-identical; dK and
    # dV take the vertical columns' contributions through fp32 atomics, whose
    # order may differ between the two runs
    assert torch.equal(ref[0], got[0]), "dQ differs"
    for name, a, b in (("dK", ref[1], got[1]), ("dV", ref[2], got[2])):
        err = float((a - b).abs().max())
        scale = float(a.abs().max())
        log(f"  {name}: max-abs {err:.3e} (max |ref| {scale:.3e})")
        assert err <= 1e-5 * max(scale, 1.0), name
    return ref


def test_bwd_noalloc_matches_bwd_twice():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dev = torch.device("cuda:0")
    _one_call(dev, 2, n=4096, v_budget=300, s_budget=1024)                       # bf16, 16 Q / 2 KV
    _one_call(dev, 1, n=1024, h_q=2, h_kv=1, d=64, v_budget=64, s_budget=128)    # fp32, smaller
