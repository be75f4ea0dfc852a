"""The C ABI on the CPU: the library loads, exports every declared symbol, and
rejects bad arguments with the documented status before any HIP call."""
import ctypes
import os
import re

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vs.h")


@pytest.fixture(scope="module")
def abi():
    from dynamic_sparse_attention_amd import _abi
    if not os.path.exists(_abi.LIB_PATH):
        from dynamic_sparse_attention_amd import build
        build.build()
    _abi.lib()
    return _abi


def declared_functions():
    text = open(HEADER).read()
    return re.findall(r"^(?:vs_status|const char\*)\s+(\w+)\s*\(", text, flags=re.M)


def test_header_symbols_exported(abi):
    names = declared_functions()
    assert set(names) == set(abi.SIGNATURES), (names, list(abi.SIGNATURES))
    L = abi.lib()
    for n in names:
        assert hasattr(L, n), n


def prob(abi, **kw):
    cu = kw.pop("cu", [0, 4096])
    arr = (ctypes.c_int32 * len(cu))(*cu)
    base = dict(batch=1, h_q=16, h_kv=2, head_dim=128, n_q=cu[-1], n_k=cu[-1], block=64,
                dtype=abi.VS_BF16, scale=0.0, n_seg=len(cu) - 1, stripe_world=1, q_rank=0, k_rank=0)
    base.update(kw)
    p = abi.VsProblem(**{k: v for k, v in base.items()})
    p.cu_seqlens = ctypes.cast(arr, abi.i32p)
    p._keep = arr
    return p


def capacity(abi, p, vb, sb):
    nl = p.batch * p.h_q * p.n_seg
    vp = (ctypes.c_int32 * (nl + 1))()
    sp = (ctypes.c_int32 * (nl + 1))()
    a = (ctypes.c_int32 * p.h_q)(*vb)
    b = (ctypes.c_int32 * p.h_q)(*sb)
    vm, sm = ctypes.c_int32(), ctypes.c_int32()
    st = abi.lib().vs_index_capacity(ctypes.byref(p), a, b, vp, sp, ctypes.byref(vm), ctypes.byref(sm))
    return st, list(vp), list(sp), vm.value, sm.value


@pytest.mark.parametrize("cu,vb,sb", [
    ([0, 131072], 2048, 8192),
    ([0, 1024], 64, 64),
    ([0, 1024], 5000, 10 ** 6),
    ([0, 640, 4096, 8192], 1000, 3000),
    ([0, 64, 128], 1, 1),
])
def test_capacity_matches_oracle(abi, cu, vb, sb):
    hq = 4
    p = prob(abi, cu=cu, h_q=hq, h_kv=1)
    vbs = [vb + h for h in range(hq)]
    sbs = [sb * (h + 1) for h in range(hq)]
    st, vp, sp, vm, sm = capacity(abi, p, vbs, sbs)
    assert st == abi.VS_OK
    for h in range(hq):
        for s in range(len(cu) - 1):
            l = h * (len(cu) - 1) + s
            kv, kg = oracle.capacities(vbs[h], sbs[h], cu[s + 1] - cu[s], cu[-1], 64)
            assert vp[l + 1] - vp[l] == kv and sp[l + 1] - sp[l] == kg
    assert vm == max(vp[i + 1] - vp[i] for i in range(len(vp) - 1))
    assert sm == max(sp[i + 1] - sp[i] for i in range(len(sp) - 1))


def test_capacity_golden(abi):
    """vs_index_capacity against the hand-derived per-document shares of
    tests/golden/segment_capacities.json (not against the oracle's function)."""
    import json
    import os
    with open(os.path.join(os.path.dirname(__file__), "golden", "segment_capacities.json")) as f:
        fx = json.load(f)
    cu = fx["cu_seqlens"]
    for case in fx["cases"]:
        p = prob(abi, cu=cu, h_q=1, h_kv=1)
        st, vp, sp, _, _ = capacity(abi, p, [case["v_budget"]], [case["s_budget"]])
        assert st == abi.VS_OK
        got = [[vp[s + 1] - vp[s], sp[s + 1] - sp[s]] for s in range(len(cu) - 1)]
        assert got == case["expected"], (case, got)


def status_of(abi, p, vb=None, sb=None):
    return capacity(abi, p, vb or [1] * p.h_q, sb or [1] * p.h_q)[0]


def test_problem_validation(abi):
    L = abi.lib()
    assert L.vs_index_capacity(None, None, None, None, None, None, None) == abi.VS_ERR_NULL
    assert "NULL" in L.vs_last_error().decode()
    assert status_of(abi, prob(abi, h_q=6, h_kv=4)) == abi.VS_ERR_SHAPE
    assert status_of(abi, prob(abi, head_dim=96)) == abi.VS_ERR_UNSUPPORTED
    assert status_of(abi, prob(abi, block=32)) == abi.VS_ERR_UNSUPPORTED
    assert status_of(abi, prob(abi, dtype=7)) == abi.VS_ERR_UNSUPPORTED
    assert status_of(abi, prob(abi, cu=[0, 100])) == abi.VS_ERR_UNSUPPORTED
    assert status_of(abi, prob(abi, cu=[64, 128])) == abi.VS_ERR_SHAPE
    assert status_of(abi, prob(abi, cu=[0, 128, 128])) == abi.VS_ERR_SHAPE
    assert status_of(abi, prob(abi, n_q=2048)) == abi.VS_ERR_SHAPE
    assert status_of(abi, prob(abi, batch=0)) == abi.VS_ERR_SHAPE
    assert status_of(abi, prob(abi, h_q=16), [-1] * 16) == abi.VS_ERR_BUDGET
    assert status_of(abi, prob(abi, scale=float("nan"))) == abi.VS_ERR_SHAPE
    many = list(range(0, 64 * 130, 64))
    assert status_of(abi, prob(abi, cu=many)) == abi.VS_ERR_UNSUPPORTED
    # bf16 K rows of one sequence are addressed with 32-bit byte offsets:
    # 2^24 tokens x 2 KV heads x 128 x 2 bytes = 8 GiB is refused, fp32 (other
    # kernels) and 2^23 tokens with one KV head (exactly 2^31 bytes) are not
    big = [0, 1 << 22, 2 << 22, 3 << 22, 4 << 22]
    assert status_of(abi, prob(abi, cu=big)) == abi.VS_ERR_UNSUPPORTED
    assert "4 GiB" in L.vs_last_error().decode()
    assert status_of(abi, prob(abi, cu=big, dtype=abi.VS_F32)) == abi.VS_OK
    assert status_of(abi, prob(abi, cu=big[:3], h_q=1, h_kv=1)) == abi.VS_OK
    # block striping
    assert status_of(abi, prob(abi, cu=[0, 8192], n_q=1024, n_k=1024, stripe_world=8, q_rank=1,
                               k_rank=7)) == abi.VS_OK
    assert status_of(abi, prob(abi, cu=[0, 8192], n_q=1024, n_k=1024, stripe_world=8, q_rank=8)) == \
        abi.VS_ERR_SHAPE
    assert status_of(abi, prob(abi, cu=[0, 4096, 8192], n_q=1024, n_k=1024, stripe_world=8)) == \
        abi.VS_ERR_UNSUPPORTED
    assert status_of(abi, prob(abi, cu=[0, 8192], n_q=2048, n_k=1024, stripe_world=8)) == abi.VS_ERR_SHAPE


def test_stride_validation(abi):
    """Strides (batch, token, head) per tensor: all zero = contiguous; negative
    ones are shape errors, ones that break 16-byte rows are unsupported; for
    bf16 the K / V rows of one head must stay within 32-bit byte offsets."""
    L = abi.lib()
    n = 4096
    fused = ((16 + 2 * 2) * 128 * n, (16 + 2 * 2) * 128, 128)  # slices of a fused QKV projection
    ok = prob(abi, q_stride=fused, k_stride=fused, v_stride=fused, o_stride=(0, 0, 0),
              do_stride=(n * 16 * 256, 16 * 256, 256))
    assert status_of(abi, ok) == abi.VS_OK
    assert status_of(abi, prob(abi, k_stride=(0, -256, 128))) == abi.VS_ERR_SHAPE
    assert "negative" in L.vs_last_error().decode()
    assert status_of(abi, prob(abi, q_stride=(0, 2052, 128))) == abi.VS_ERR_UNSUPPORTED
    assert "multiple of 8" in L.vs_last_error().decode()
    assert status_of(abi, prob(abi, o_stride=(0, 2048, 132))) == abi.VS_ERR_UNSUPPORTED
    assert status_of(abi, prob(abi, do_stride=(4, 0, 0))) == abi.VS_ERR_UNSUPPORTED
    # K rows 2^20 tokens apart at a stride of 4096 elements: (2^20 - 1) * 8 KiB
    # exceeds 4 GiB of byte offsets in bf16, not in fp32 (other kernels)
    cu = [0, 1 << 20]
    wide = (0, 4096, 128)
    assert status_of(abi, prob(abi, cu=cu, k_stride=wide)) == abi.VS_ERR_UNSUPPORTED
    assert "4 GiB" in L.vs_last_error().decode()
    assert status_of(abi, prob(abi, cu=cu, v_stride=wide)) == abi.VS_ERR_UNSUPPORTED
    assert status_of(abi, prob(abi, cu=cu, k_stride=wide, dtype=abi.VS_F32)) == abi.VS_OK
    assert status_of(abi, prob(abi, cu=cu, q_stride=wide)) == abi.VS_OK  # Q rows use 64-bit offsets


def test_noalloc_backward_refuses_large_problems(abi):
    """vs_sparse_attn_bwd_noalloc refuses a problem whose workspace exceeds the
    library's fixed array, before any HIP call (so also without a GPU)."""
    L = abi.lib()
    n = 1 << 20
    p = prob(abi, cu=[0, n], h_q=32, h_kv=4)   # delta and LSE rows alone: 2 * 32 * 2^20 * 4 B = 256 MiB
    ix = abi.VsIndex(0x1000, 0x1000, 0x1000, 0x1000, 64, 4)
    nb = ctypes.c_size_t()
    assert L.vs_workspace_size(ctypes.byref(p), 2, ctypes.byref(ix), ctypes.byref(nb)) == abi.VS_OK
    assert nb.value > 64 << 20
    st = L.vs_sparse_attn_bwd_noalloc(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, 0, FAKE, FAKE, None,
                                      ctypes.byref(ix), FAKE, 0, FAKE, FAKE, None)
    assert st == abi.VS_ERR_WORKSPACE
    assert "fixed" in L.vs_last_error().decode()
    # argument errors come first, as in vs_sparse_attn_bwd
    st = L.vs_sparse_attn_bwd_noalloc(ctypes.byref(p), None, FAKE, FAKE, FAKE, 0, FAKE, FAKE, None,
                                      ctypes.byref(ix), FAKE, 0, FAKE, FAKE, None)
    assert st == abi.VS_ERR_NULL


def test_all_chunks_validation(abi):
    """k_rank = VS_ALL_CHUNKS: K / V hold every rank's chunk, so n_k = n_global."""
    W = 8
    kw = dict(cu=[0, 8192], n_q=1024, stripe_world=W, q_rank=3, k_rank=abi.VS_ALL_CHUNKS)
    assert status_of(abi, prob(abi, n_k=8192, **kw)) == abi.VS_OK
    assert status_of(abi, prob(abi, n_k=1024, **kw)) == abi.VS_ERR_SHAPE
    assert status_of(abi, prob(abi, n_k=8192, **dict(kw, k_rank=-2))) == abi.VS_ERR_SHAPE
    # without striping the field is ignored (one contiguous sequence)
    assert status_of(abi, prob(abi, k_rank=abi.VS_ALL_CHUNKS)) == abi.VS_OK


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation first


def test_entry_points_reject_before_launch(abi):
    L = abi.lib()
    p = prob(abi)
    P = ctypes.byref(p)
    ix = abi.VsIndex(0x1000, 0x1000, 0x1000, 0x1000, 64, 4)
    nb = ctypes.c_size_t()
    assert L.vs_workspace_size(P, 0, None, ctypes.byref(nb)) == abi.VS_OK and nb.value > 0
    assert L.vs_workspace_size(P, 1, ctypes.byref(ix), ctypes.byref(nb)) == abi.VS_OK
    fwd_ws = nb.value
    assert L.vs_workspace_size(P, 2, ctypes.byref(ix), ctypes.byref(nb)) == abi.VS_OK
    assert nb.value > fwd_ws
    assert L.vs_workspace_size(P, 5, ctypes.byref(ix), ctypes.byref(nb)) == abi.VS_ERR_SHAPE
    assert L.vs_workspace_size(P, 1, None, ctypes.byref(nb)) == abi.VS_ERR_NULL
    # estimate
    st = L.vs_estimate_index(P, FAKE, FAKE, 32, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, 1 << 40, None)
    assert st == abi.VS_ERR_UNSUPPORTED
    st = L.vs_estimate_index(P, FAKE, FAKE, 0, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, 16, None)
    assert st == abi.VS_ERR_WORKSPACE
    st = L.vs_estimate_index(P, None, FAKE, 0, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, 1 << 40, None)
    assert st == abi.VS_ERR_NULL
    ps = prob(abi, cu=[0, 8192], n_q=1024, n_k=1024, stripe_world=8)
    st = L.vs_estimate_index(ctypes.byref(ps), FAKE, FAKE, 0, FAKE, FAKE, FAKE, FAKE, None, None, FAKE,
                             1 << 40, None)
    assert st == abi.VS_ERR_UNSUPPORTED
    # estimate with top-p budgets
    st = L.vs_estimate_index_topp(P, FAKE, FAKE, 0, None, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None,
                                  FAKE, 1 << 40, None)
    assert st == abi.VS_ERR_NULL
    st = L.vs_estimate_index_topp(P, FAKE, FAKE, 32, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None,
                                  FAKE, 1 << 40, None)
    assert st == abi.VS_ERR_UNSUPPORTED
    st = L.vs_estimate_index_topp(P, FAKE, FAKE, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None,
                                  FAKE, 16, None)
    assert st == abi.VS_ERR_WORKSPACE
    # forward
    st = L.vs_sparse_attn_fwd(P, FAKE, FAKE, FAKE, ctypes.byref(ix), FAKE, 0, FAKE, FAKE, 16, None)
    assert st == abi.VS_ERR_WORKSPACE
    st = L.vs_sparse_attn_fwd(P, FAKE, FAKE, FAKE, ctypes.byref(ix), FAKE, 3, FAKE, FAKE, 1 << 40, None)
    assert st == abi.VS_ERR_SHAPE  # o_f32 is 0, 1 or 2 (merge into the running result)
    st = L.vs_sparse_attn_fwd(P, FAKE, FAKE, None, ctypes.byref(ix), FAKE, 0, FAKE, FAKE, 1 << 40, None)
    assert st == abi.VS_ERR_NULL
    bad = abi.VsIndex(0x1000, 0x1000, 0x1000, 0x1000, 5000, 4)
    st = L.vs_sparse_attn_fwd(P, FAKE, FAKE, FAKE, ctypes.byref(bad), FAKE, 0, FAKE, FAKE, 1 << 40, None)
    assert st == abi.VS_ERR_INDEX
    bad = abi.VsIndex(0x1000, 0x1000, 0x1000, 0x1000, 64, 65)
    st = L.vs_sparse_attn_fwd(P, FAKE, FAKE, FAKE, ctypes.byref(bad), FAKE, 0, FAKE, FAKE, 1 << 40, None)
    assert st == abi.VS_ERR_INDEX
    bad = abi.VsIndex(0x1000, None, 0x1000, 0x1000, 64, 4)
    st = L.vs_sparse_attn_fwd(P, FAKE, FAKE, FAKE, ctypes.byref(bad), FAKE, 0, FAKE, FAKE, 1 << 40, None)
    assert st == abi.VS_ERR_NULL
    # backward
    st = L.vs_sparse_attn_bwd(P, FAKE, FAKE, FAKE, None, 0, FAKE, FAKE, None, ctypes.byref(ix), FAKE, 0,
                              FAKE, FAKE, FAKE, 1 << 40, None)
    assert st == abi.VS_ERR_NULL
    st = L.vs_sparse_attn_bwd(P, FAKE, FAKE, FAKE, FAKE, 0, FAKE, FAKE, None, ctypes.byref(ix), FAKE, 0,
                              FAKE, FAKE, FAKE, fwd_ws, None)
    assert st == abi.VS_ERR_WORKSPACE
    wide = prob(abi, h_q=33, h_kv=1)  # a GQA group of 33 Q heads: beyond the bf16 dK/dV tile tags
    st = L.vs_sparse_attn_bwd(ctypes.byref(wide), FAKE, FAKE, FAKE, FAKE, 0, FAKE, FAKE, None,
                              ctypes.byref(ix), FAKE, 0, FAKE, FAKE, FAKE, 1 << 40, None)
    assert st == abi.VS_ERR_UNSUPPORTED and "32 Q heads" in L.vs_last_error().decode()
    st = L.vs_attn_bwd_delta(P, None, 0, FAKE, FAKE, None)
    assert st == abi.VS_ERR_NULL
    # merge
    assert L.lse_merge(1, 16, 2, 96, FAKE, FAKE, FAKE, FAKE, None) == abi.VS_ERR_UNSUPPORTED
    assert L.lse_merge(1, 16, 2, 128, None, FAKE, FAKE, FAKE, None) == abi.VS_ERR_NULL
    assert L.lse_merge(-1, 16, 2, 128, FAKE, FAKE, FAKE, FAKE, None) == abi.VS_ERR_SHAPE


def test_executed_area_matches_oracle():
    """Host work accounting of the package equals the oracle's mask-area count."""
    import numpy as np
    from dynamic_sparse_attention_amd import accounting
    from test_oracle_pins import rand_index
    rng = np.random.default_rng(21)
    for cu in ([0, 1024], [0, 256, 640, 1024], [0, 4096]):
        n = cu[-1]
        idx = rand_index(rng, n, 3, 64, cu=cu)
        lists = [idx[(h, s)] for h in range(3) for s in range(len(cu) - 1)]
        got = accounting.executed_area(lists, cu, 3)
        assert got.tolist() == oracle.mask_area_formula(cu, idx, 3)
        pos = np.arange(n)
        assert accounting.dense_causal_area(cu) == oracle.dense_causal_area(pos, cu)
    # a block-striped worker's rows
    n, W, w = 2048, 4, 1
    idx = rand_index(rng, n, 2, 64, kv=50, kg=5)
    rows_b = np.arange(w, n // 64, W)
    rows = (rows_b[:, None] * 64 + np.arange(64)).reshape(-1)
    lists = [idx[(h, 0)] for h in range(2)]
    got = accounting.executed_area(lists, [0, n], 2, row_blocks=rows_b)
    ref = [int(oracle.dense_mask(rows, np.arange(n), [0, n], idx, h).sum()) for h in range(2)]
    assert got.tolist() == ref
    assert accounting.dense_causal_area([0, n], rows) == oracle.dense_causal_area(rows, [0, n])
    # a block selection (128-token blocks, ragged last block): the oracle's mask count
    n, nI = 128 * 5 + 64, 6
    sel = (rng.random((2, nI, nI)) < 0.5) & np.tril(np.ones((nI, nI), bool))
    e = np.zeros(0, np.int64)
    bidx = {(h, 0): (e, e, (128, sel[h])) for h in range(2)}
    pos = np.arange(n)
    ref = [int(oracle.dense_mask(pos, pos, [0, n], bidx, h).sum()) for h in range(2)]
    assert accounting.block_selection_area(sel, n).tolist() == ref
    # a per-row selection (blocks of 32 tokens, a short last block): the oracle's mask count
    n, blk = 32 * 5 + 16, 32
    nB = 6
    own = np.arange(n) // blk
    rsel = (rng.random((2, n, nB)) < 0.5) & (np.arange(nB)[None, None, :] <= own[None, :, None])
    ridx = {(h, 0): (e, e, None, (blk, rsel[h])) for h in range(2)}
    pos = np.arange(n)
    ref = [int(oracle.dense_mask(pos, pos, [0, n], ridx, h).sum()) for h in range(2)]
    words = (rsel * (1 << np.arange(nB))[None, None, :]).sum(axis=-1)
    assert accounting.row_selection_area(words, n, blk).tolist() == ref


def test_xattn_and_block_selection_validation(abi):
    """The XAttention estimator and a block-selection index: supported forms
    (bf16, one segment, no striping, 128-token blocks, stride 16, at most
    1024 query blocks) are checked before any HIP call."""
    L = abi.lib()
    p = prob(abi)
    P = ctypes.byref(p)
    nb = ctypes.c_size_t()
    assert L.vs_workspace_size(P, 3, None, ctypes.byref(nb)) == abi.VS_OK
    nC, nI = 4096 // 16, 4096 // 128
    assert nb.value >= 16 * nC * nI * 4   # (key block, cell row) log-sum-exps, fp32
    big = 1 << 40
    est = L.vs_estimate_index_xattn
    assert est(P, None, FAKE, 128, 16, 0.9, FAKE, None, None, FAKE, big, None) == abi.VS_ERR_NULL
    assert est(P, FAKE, FAKE, 128, 16, 0.9, None, None, None, FAKE, big, None) == abi.VS_ERR_NULL
    assert est(P, FAKE, FAKE, 64, 16, 0.9, FAKE, None, None, FAKE, big, None) == abi.VS_ERR_UNSUPPORTED
    assert est(P, FAKE, FAKE, 128, 8, 0.9, FAKE, None, None, FAKE, big, None) == abi.VS_ERR_UNSUPPORTED
    assert est(P, FAKE, FAKE, 128, 16, float("nan"), FAKE, None, None, FAKE, big, None) == abi.VS_ERR_SHAPE
    assert est(P, FAKE, FAKE, 128, 16, 0.9, FAKE, None, None, FAKE, 16, None) == abi.VS_ERR_WORKSPACE
    for bad in (prob(abi, dtype=abi.VS_F32), prob(abi, cu=[0, 2048, 4096]),
                prob(abi, cu=[0, 8192], n_q=1024, n_k=1024, stripe_world=8),
                prob(abi, cu=[0, 131072 + 128])):
        assert est(ctypes.byref(bad), FAKE, FAKE, 128, 16, 0.9, FAKE, None, None, FAKE, big,
                   None) == abi.VS_ERR_UNSUPPORTED
    # a block-selection index
    ix = abi.VsIndex(0x1000, 0x1000, 0x1000, 0x1000, 0, 0, 0x1000, 128)
    assert L.vs_workspace_size(P, 1, ctypes.byref(ix), ctypes.byref(nb)) == abi.VS_OK
    for bad_ix in (abi.VsIndex(0x1000, 0x1000, 0x1000, 0x1000, 0, 0, 0x1000, 64),
                   abi.VsIndex(0x1000, 0x1000, 0x1000, 0x1000, 0, 0, 0x1000, 256)):
        assert L.vs_workspace_size(P, 1, ctypes.byref(bad_ix), ctypes.byref(nb)) == abi.VS_ERR_UNSUPPORTED
    lists = abi.VsIndex(0x1000, 0x1000, 0x1000, 0x1000, 64, 4, 0x1000, 128)
    assert L.vs_workspace_size(P, 2, ctypes.byref(lists), ctypes.byref(nb)) == abi.VS_ERR_INDEX
    for bad in (prob(abi, dtype=abi.VS_F32), prob(abi, cu=[0, 2048, 4096])):
        assert L.vs_workspace_size(ctypes.byref(bad), 1, ctypes.byref(ix),
                                   ctypes.byref(nb)) == abi.VS_ERR_UNSUPPORTED


def test_moba_and_row_selection_validation(abi):
    """The MoBA gate and a per-row block selection: supported forms (bf16,
    one segment, no striping, a power-of-two block of at least 256 tokens
    for the gate and 64 for the index, at most 32 blocks) are checked before
    any HIP call."""
    L = abi.lib()
    p = prob(abi, cu=[0, 8192])
    P = ctypes.byref(p)
    nb = ctypes.c_size_t()
    assert L.vs_workspace_size(P, 4, None, ctypes.byref(nb)) == abi.VS_OK
    assert nb.value >= 2 * 32 * 128 * 4        # the blocks' mean keys, fp32, room for 32 blocks
    big = 1 << 40
    est = L.vs_estimate_index_moba
    assert est(P, None, FAKE, 512, 4, FAKE, None, FAKE, big, None) == abi.VS_ERR_NULL
    assert est(P, FAKE, FAKE, 512, 4, None, None, FAKE, big, None) == abi.VS_ERR_NULL
    assert est(P, FAKE, FAKE, 128, 4, FAKE, None, FAKE, big, None) == abi.VS_ERR_UNSUPPORTED   # block < 256
    assert est(P, FAKE, FAKE, 768, 4, FAKE, None, FAKE, big, None) == abi.VS_ERR_UNSUPPORTED   # not a power of 2
    p64 = prob(abi, cu=[0, 16384])              # 64 blocks of 256: beyond the 32 a row's word holds
    assert est(ctypes.byref(p64), FAKE, FAKE, 256, 4, FAKE, None, FAKE, big, None) == abi.VS_ERR_UNSUPPORTED
    assert est(P, FAKE, FAKE, 512, 0, FAKE, None, FAKE, big, None) == abi.VS_ERR_SHAPE
    assert est(P, FAKE, FAKE, 512, 4, FAKE, None, FAKE, 16, None) == abi.VS_ERR_WORKSPACE
    for bad in (prob(abi, dtype=abi.VS_F32, cu=[0, 8192]), prob(abi, cu=[0, 4096, 8192]),
                prob(abi, cu=[0, 8192], n_q=1024, n_k=1024, stripe_world=8)):
        assert est(ctypes.byref(bad), FAKE, FAKE, 512, 4, FAKE, None, FAKE, big, None) == abi.VS_ERR_UNSUPPORTED
    # a per-row selection in the index
    ix = abi.VsIndex(0x1000, 0x1000, 0x1000, 0x1000, 0, 0, None, 0, 0x1000, 512)
    assert L.vs_workspace_size(P, 2, ctypes.byref(ix), ctypes.byref(nb)) == abi.VS_OK
    for rb in (32, 96, 128):                    # below 64, not a power of 2, 64 blocks at n = 8192
        bad_ix = abi.VsIndex(0x1000, 0x1000, 0x1000, 0x1000, 0, 0, None, 0, 0x1000, rb)
        assert L.vs_workspace_size(P, 1, ctypes.byref(bad_ix), ctypes.byref(nb)) == abi.VS_ERR_UNSUPPORTED
    both = abi.VsIndex(0x1000, 0x1000, 0x1000, 0x1000, 0, 0, 0x1000, 128, 0x1000, 512)
    assert L.vs_workspace_size(P, 1, ctypes.byref(both), ctypes.byref(nb)) == abi.VS_ERR_INDEX
    lists = abi.VsIndex(0x1000, 0x1000, 0x1000, 0x1000, 64, 4, None, 0, 0x1000, 512)
    assert L.vs_workspace_size(P, 2, ctypes.byref(lists), ctypes.byref(nb)) == abi.VS_ERR_INDEX
    for bad in (prob(abi, dtype=abi.VS_F32, cu=[0, 8192]), prob(abi, cu=[0, 4096, 8192])):
        assert L.vs_workspace_size(ctypes.byref(bad), 1, ctypes.byref(ix),
                                   ctypes.byref(nb)) == abi.VS_ERR_UNSUPPORTED
