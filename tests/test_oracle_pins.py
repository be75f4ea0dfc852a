"""Pins of the CPU oracle against facts the pages and mathematics fix (no GPU).

Each test names the passage or the mathematical fact that fixes the expected
value, so that a slip in the oracle (a dropped term, a wrong sign, index or
operand) fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import rope as orope

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_index(rng, n, hq, block, cu=None, kv=None, kg=None):
    """Random (not estimated) Vertical-Slash index for every (head, segment)."""
    cu = cu or [0, n]
    idx = {}
    for h in range(hq):
        for s in range(len(cu) - 1):
            a, e = cu[s], cu[s + 1]
            L = e - a
            nb = -(-L // block)
            nv = rng.integers(0, L + 1) if kv is None else min(kv, L)
            ng = rng.integers(0, nb + 1) if kg is None else min(kg, nb)
            iv = np.sort(rng.choice(L, size=nv, replace=False)) + a
            is_ = np.sort(rng.choice(nb, size=ng, replace=False))
            idx[(h, s)] = (iv.astype(np.int64), is_.astype(np.int64))
    return idx


def full_index(n, hq, block, cu=None):
    cu = cu or [0, n]
    return {(h, s): (np.zeros(0, np.int64), np.arange(-(-(cu[s + 1] - cu[s]) // block)))
            for h in range(hq) for s in range(len(cu) - 1)}


def triple_loop_causal(q, k, v, scale):
    """Textbook causal softmax attention, scalar Python loops (one head)."""
    n, d = q.shape
    out = np.zeros_like(v)
    lse = np.zeros(n)
    for i in range(n):
        s = [scale * sum(q[i, c] * k[j, c] for c in range(d)) for j in range(i + 1)]
        mx = max(s)
        z = sum(math.exp(x - mx) for x in s)
        lse[i] = mx + math.log(z)
        for j in range(i + 1):
            p = math.exp(s[j] - lse[i])
            out[i] += p * v[j]
    return out, lse


# ---------------------------------------------------------------- P1 brute force
def test_p1_all_blocks_equals_dense_causal():
    """All block-diagonals selected gives plain causal attention (Algorithm 1 mask)."""
    rng = np.random.default_rng(1)
    n, d, B = 48, 8, 16
    q, k, v = (rng.standard_normal((n, 1, d)) for _ in range(3))
    pos = np.arange(n)
    O, L = oracle.attn_fwd_dense(q, k, v, pos, pos, [0, n], full_index(n, 1, B), B)
    O2, L2 = triple_loop_causal(q[:, 0], k[:, 0], v[:, 0], 1 / math.sqrt(d))
    assert np.abs(O[:, 0] - O2).max() < 1e-12
    assert np.abs(L[0] - L2).max() < 1e-12
    # the same with every vertical selected and no slash
    idx = {(0, 0): (np.arange(n), np.zeros(0, np.int64))}
    O3, L3 = oracle.attn_fwd_dense(q, k, v, pos, pos, [0, n], idx, B)
    assert np.abs(O3 - O).max() < 1e-12 and np.abs(L3 - L).max() < 1e-12


def test_p1_gqa_fwd_bwd_equals_torch_sdpa():
    """Full index, GQA: forward and gradients equal torch's causal SDPA in fp64 on CPU."""
    rng = np.random.default_rng(2)
    n, hq, hkv, d, B = 128, 4, 2, 16, 32
    q, do = rng.standard_normal((n, hq, d)), rng.standard_normal((n, hq, d))
    k, v = rng.standard_normal((n, hkv, d)), rng.standard_normal((n, hkv, d))
    pos = np.arange(n)
    idx = full_index(n, hq, B)
    O, L = oracle.attn_fwd_dense(q, k, v, pos, pos, [0, n], idx, B)
    D = oracle.bwd_delta(O, do)
    assert np.abs(D - (O * do).sum(-1).T).max() < 1e-15
    dq, dk, dv = oracle.attn_bwd_dense(q, k, v, do, L, D, pos, pos, [0, n], idx, B)
    tq = torch.tensor(q).permute(1, 0, 2).requires_grad_()
    tk = torch.tensor(k).permute(1, 0, 2).requires_grad_()
    tv = torch.tensor(v).permute(1, 0, 2).requires_grad_()
    kk = tk.repeat_interleave(hq // hkv, 0)
    vv = tv.repeat_interleave(hq // hkv, 0)
    to = torch.nn.functional.scaled_dot_product_attention(tq, kk, vv, is_causal=True)
    to.backward(torch.tensor(do).permute(1, 0, 2))
    assert np.abs(to.detach().permute(1, 0, 2).numpy() - O).max() < 1e-12
    assert np.abs(tq.grad.permute(1, 0, 2).numpy() - dq).max() < 1e-12
    assert np.abs(tk.grad.permute(1, 0, 2).numpy() - dk).max() < 1e-12
    assert np.abs(tv.grad.permute(1, 0, 2).numpy() - dv).max() < 1e-12


# ---------------------------------------------------------------- P2 special case
def test_p2_diagonal_only_is_block_local_causal():
    """I_s = {0}, no verticals: each block is an independent causal attention."""
    rng = np.random.default_rng(3)
    n, d, B = 96, 8, 32
    q, k, v = (rng.standard_normal((n, 1, d)) for _ in range(3))
    pos = np.arange(n)
    idx = {(0, 0): (np.zeros(0, np.int64), np.array([0]))}
    O, L = oracle.attn_fwd_dense(q, k, v, pos, pos, [0, n], idx, B)
    for b in range(n // B):
        sl = slice(b * B, (b + 1) * B)
        t = torch.nn.functional.scaled_dot_product_attention(
            torch.tensor(q[sl, 0])[None], torch.tensor(k[sl, 0])[None], torch.tensor(v[sl, 0])[None],
            is_causal=True)[0].numpy()
        assert np.abs(O[sl, 0] - t).max() < 1e-12


# ---------------------------------------------------------------- P3 closed forms
def test_p3_zero_query_hand_derived_mask():
    """Q = 0 makes every score 0: LSE[n] = ln|M_n|, O[n] = mean of V over the row's support.

    The support sizes come from the fixture, derived by hand from the mask
    definition (causal and (selected column or selected block-diagonal)).
    """
    with open(os.path.join(GOLDEN, "zero_query_mask.json")) as f:
        fx = json.load(f)
    n, B, d = fx["n"], fx["block"], 4
    idx = {(0, 0): (np.array(fx["verticals"]), np.array(fx["slashes"]))}
    rng = np.random.default_rng(4)
    q = np.zeros((n, 1, d))
    k, v, do = (rng.standard_normal((n, 1, d)) for _ in range(3))
    pos = np.arange(n)
    O, L = oracle.attn_fwd_dense(q, k, v, pos, pos, [0, n], idx, B)
    O2, L2 = oracle.attn_fwd_support(q, k, v, pos, pos, [0, n], idx, B)
    sizes = np.zeros(n, np.int64)
    for lo, hi, cnt in fx["row_support_sizes"]:
        sizes[lo:hi] = cnt
    # rows that see column 130 only from n >= 130 on
    for r in fx["plus_one_from"]:
        sizes[r[0]:r[1]] += np.arange(r[1] - r[0]) >= (r[2] - r[0])
    emp = sizes == 0
    assert np.all(np.isneginf(L[0, emp])) and np.all(O[emp] == 0)
    assert np.abs(L[0, ~emp] - np.log(sizes[~emp])).max() < 1e-12
    assert np.allclose(L2, L, atol=1e-12, equal_nan=False) or np.array_equal(L2, L)
    M = oracle.dense_mask(pos, pos, [0, n], idx, 0, B)
    assert np.array_equal(M.sum(1), sizes)
    mean_v = (M.astype(float) @ v[:, 0]) / np.maximum(sizes, 1)[:, None]
    assert np.abs(O[:, 0] - mean_v).max() < 1e-12
    # dV[m] = sum over rows n that see m of dO[n] / |M_n| (Eq. 2 with A = M / |M_n|)
    D = (O * do).sum(-1).T
    _, _, dv = oracle.attn_bwd_dense(q, k, v, do, L, D, pos, pos, [0, n], idx, B)
    w = M / np.maximum(sizes, 1)[:, None]
    assert np.abs(dv[:, 0] - w.T @ do[:, 0]).max() < 1e-12


# ---------------------------------------------------------------- P4 finite differences
def test_p4_finite_differences_and_delta_identity():
    """Gradients of L = sum(O * dO) wrt Q, K, V by central differences (index fixed)."""
    rng = np.random.default_rng(5)
    n, hq, hkv, d, B = 64, 2, 1, 8, 16
    q, do = rng.standard_normal((n, hq, d)), rng.standard_normal((n, hq, d))
    k, v = rng.standard_normal((n, hkv, d)), rng.standard_normal((n, hkv, d))
    pos = np.arange(n)
    idx = rand_index(rng, n, hq, B, kv=6, kg=2)
    O, L = oracle.attn_fwd_dense(q, k, v, pos, pos, [0, n], idx, B)
    D = (O * do).sum(-1).T
    dq, dk, dv = oracle.attn_bwd_dense(q, k, v, do, L, D, pos, pos, [0, n], idx, B)

    def loss(qq, kk, vv):
        o, _ = oracle.attn_fwd_dense(qq, kk, vv, pos, pos, [0, n], idx, B)
        return (o * do).sum()

    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        flat = x.reshape(-1)
        picks = rng.choice(flat.size, size=40, replace=False)
        for p in picks:
            xp, xm = flat.copy(), flat.copy()
            xp[p] += h
            xm[p] -= h
            args = {"q": q, "k": k, "v": v}
            args[name] = xp.reshape(x.shape)
            lp = loss(args["q"], args["k"], args["v"])
            args[name] = xm.reshape(x.shape)
            lm = loss(args["q"], args["k"], args["v"])
            fd = (lp - lm) / (2 * h)
            assert abs(fd - g.reshape(-1)[p]) <= 1e-6 * max(1.0, abs(fd)), (name, p)
    # D = rowsum(dA * A) (Eq. 1) equals rowsum(dO * O)
    for hh in range(hq):
        M = oracle.dense_mask(pos, pos, [0, n], idx, hh, B)
        S = np.where(M, (q[:, hh] @ k[:, 0].T) / math.sqrt(d), -np.inf)
        A = np.where(M, np.exp(S - np.where(np.isfinite(L[hh]), L[hh], 0)[:, None]), 0)
        dA = do[:, hh] @ v[:, 0].T
        assert np.abs((dA * A).sum(1) - D[hh]).max() < 1e-12


# ---------------------------------------------------------------- P5 exact merge identity
def test_p5_lse_merge_identity_over_random_partitions():
    rng = np.random.default_rng(6)
    n, hq, d, B = 128, 2, 8, 32
    q = rng.standard_normal((n, hq, d))
    k, v = rng.standard_normal((n, 1, d)), rng.standard_normal((n, 1, d))
    pos = np.arange(n)
    idx = rand_index(rng, n, hq, B, kv=20, kg=2)
    O, L = oracle.attn_fwd_dense(q, k, v, pos, pos, [0, n], idx, B)
    for nchunks in (2, 5, 32):
        owner = rng.integers(0, nchunks, size=n)
        acc_o = np.zeros((hq, n, d))
        acc_l = np.full((hq, n), -np.inf)
        for c in rng.permutation(nchunks):
            cols = np.nonzero(owner == c)[0]
            o, l = oracle.attn_fwd_dense(q, k[cols], v[cols], pos, cols, [0, n], idx, B)
            acc_o, acc_l = oracle.lse_merge(acc_o, acc_l, o.transpose(1, 0, 2), l)
        fin = np.isfinite(L)
        assert np.array_equal(np.isneginf(acc_l), ~fin)
        assert np.abs(acc_l[fin] - L[fin]).max() < 1e-12
        assert np.abs(acc_o - O.transpose(1, 0, 2)).max() < 1e-12


def test_p5_merge_algebra():
    rng = np.random.default_rng(7)
    o = [rng.standard_normal((5, 3)) for _ in range(3)]
    l = [rng.standard_normal(5) * 4 for _ in range(3)]
    l[1][2] = -np.inf
    o[1][2] = 0
    a = oracle.lse_merge(*oracle.lse_merge(o[0], l[0], o[1], l[1]), o[2], l[2])
    b = oracle.lse_merge(o[0], l[0], *oracle.lse_merge(o[1], l[1], o[2], l[2]))
    c = oracle.lse_merge(o[1], l[1], o[0], l[0])
    d_ = oracle.lse_merge(o[0], l[0], o[1], l[1])
    assert np.allclose(a[0], b[0], atol=1e-14) and np.allclose(a[1], b[1], atol=1e-14)
    assert np.array_equal(c[1], d_[1]) and np.allclose(c[0], d_[0], atol=1e-15)
    e = oracle.lse_merge(o[0], l[0], np.zeros((5, 3)), np.full(5, -np.inf))
    assert np.array_equal(e[1], l[0]) and np.allclose(e[0], o[0], atol=1e-15)
    z = oracle.lse_merge(np.zeros((5, 3)), np.full(5, -np.inf), np.zeros((5, 3)), np.full(5, -np.inf))
    assert np.all(np.isneginf(z[1])) and np.all(z[0] == 0)
    # two halves of one softmax: log-add-exp of the halves' sums
    s = rng.standard_normal(10)
    vv = rng.standard_normal((10, 3))
    def part(ix):
        m = s[ix].max()
        p = np.exp(s[ix] - m)
        return (p @ vv[ix]) / p.sum(), m + np.log(p.sum())
    o1, l1 = part(np.arange(4))
    o2, l2 = part(np.arange(4, 10))
    om, lm = oracle.lse_merge(o1[None], np.array([l1]), o2[None], np.array([l2]))
    p = np.exp(s - s.max())
    assert abs(lm[0] - (s.max() + np.log(p.sum()))) < 1e-14
    assert np.abs(om[0] - (p @ vv) / p.sum()).max() < 1e-14


# ---------------------------------------------------------------- P6 tie pins / selection
def test_p6_zero_query_ties_go_to_lowest_index():
    """Q = 0: every window row is uniform over its causal keys, so v[m] is equal for
    all m up to the first window row and sigma[g] is equal for g >= 1 (sigma[0] smaller)."""
    rng = np.random.default_rng(8)
    n, d, B = 512, 8, 64
    q = np.zeros((n, 1, d))
    k = rng.standard_normal((n, 1, d))
    idx, sc = oracle.estimate_index(q, k, [0, n], [100], [3 * B], B, 64, return_scores=True)
    iv, is_ = idx[(0, 0)]
    assert np.array_equal(iv, np.arange(100))
    assert np.array_equal(is_, np.array([1, 2, 3]))
    v, sigma = sc[(0, 0)]
    assert np.all(v[: n - 63] == v[0]) and np.all(v[n - 63:] < v[0])
    assert np.allclose(sigma[1:], sigma[1]) and sigma[0] < sigma[1]


def test_p6_duplicate_keys_lower_index_wins():
    rng = np.random.default_rng(9)
    n, d, B = 256, 8, 64
    q = rng.standard_normal((n, 1, d))
    k = rng.standard_normal((n, 1, d))
    k[40] = k[7] * 5
    k[7] = k[7] * 5
    _, sc = oracle.estimate_index(q, k, [0, n], [1], [0], B, 64, return_scores=True)
    v, _ = sc[(0, 0)]
    assert v[7] == v[40]
    kmax = int(np.argmax(v))
    assert kmax == 7
    idx = oracle.estimate_index(q, k, [0, n], [1], [0], B, 64)
    assert idx[(0, 0)][0].tolist() == [7]


def test_p6_topk_matches_stable_sort():
    rng = np.random.default_rng(10)
    for _ in range(50):
        x = rng.integers(0, 6, size=40).astype(float)
        kk = int(rng.integers(0, 41))
        ref = sorted(sorted(range(40), key=lambda i: (-x[i], i))[:kk])
        assert oracle.select_topk(x, kk).tolist() == ref


# ---------------------------------------------------------------- top-p budgets (Algorithm 1 topp)
def test_topp_brute_force_over_subsets():
    """topp(x, p) is the size of the smallest subset whose mass reaches p of the
    total (MTraining §4.1 (i): the minimal number of lines that recall a target
    proportion of the mass) — found here by enumerating every subset."""
    import itertools
    rng = np.random.default_rng(21)
    for _ in range(200):
        n = int(rng.integers(1, 8))
        x = rng.integers(0, 5, size=n).astype(float) * rng.choice([1.0, 0.37])
        p = float(rng.choice([0.0, 0.1, 0.33, 0.5, 0.8, 0.95, 1.0, rng.random()]))
        total = x.sum()
        best = 0
        if p > 0 and total > 0:
            best = min(len(c) for r in range(1, n + 1) for c in itertools.combinations(range(n), r)
                       if sum(x[list(c)]) >= p * total)
        assert oracle.topp_count(x, p) == best, (x, p)


def test_topp_closed_forms():
    """Uniform masses need ceil(p n) entries; geometric masses r^i need
    ceil(log(1 - p (1 - r^n)) / log r) (partial sums of a geometric series);
    p <= 0 or zero mass gives 0, p >= 1 every positive entry."""
    rng = np.random.default_rng(22)
    for n in (1, 7, 64, 1000):
        for p in (0.01, 0.25, 0.5, 0.9, 0.999):
            assert oracle.topp_count(np.full(n, 0.125), p) == math.ceil(p * n - 1e-12)
    for r in (0.5, 0.9, 0.99):
        n = 300
        x = r ** np.arange(n)
        perm = rng.permutation(n)  # positions do not matter, only the masses
        for p in (0.1, 0.37, 0.6, 0.9, 0.99):
            t = math.log(1 - p * (1 - r ** n)) / math.log(r)
            if abs(t - round(t)) < 1e-6:
                continue
            assert oracle.topp_count(x[perm], p) == math.ceil(t), (r, p)
    x = np.array([0.0, 3.0, 0.0, 1.0, 2.0])
    assert oracle.topp_count(x, 0.0) == 0 and oracle.topp_count(x, -1.0) == 0
    assert oracle.topp_count(x, 1.0) == 3 and oracle.topp_count(x, 2.0) == 3
    assert oracle.topp_count(np.zeros(9), 0.5) == 0


def test_topp_index_reduces_to_fixed_budgets():
    """With p = 1 and budgets at or below the number of positive scores, the
    top-p index is the fixed-budget index (argtopk with those budgets); with
    p = 1 and unbounded budgets every positive-mass candidate is selected."""
    rng = np.random.default_rng(23)
    n, hq, hkv, d, B = 640, 2, 1, 16, 64
    q = rng.standard_normal((n, hq, d))
    k = rng.standard_normal((n, hkv, d))
    cu = [0, 256, n]
    vb, sb = [70, 40], [200, 130]
    fixed = oracle.estimate_index(q, k, cu, vb, sb, B, 64)
    topp, sc, cnt = oracle.estimate_index_topp(q, k, cu, vb, sb, [1.0, 1.0], [1.0, 1.0], B, 64,
                                               return_scores=True)
    for key in fixed:
        assert np.array_equal(fixed[key][0], topp[key][0]) and np.array_equal(fixed[key][1], topp[key][1])
    big, sc, cnt = oracle.estimate_index_topp(q, k, cu, [n] * hq, [n] * hq, [1.0] * hq, [1.0] * hq, B, 64,
                                              return_scores=True)
    for (h, s), (iv, is_) in big.items():
        v, sigma = sc[(h, s)]
        assert iv.size == int(np.count_nonzero(v > 0)) and is_.size == int(np.count_nonzero(sigma > 0))
        # and a smaller p keeps a prefix of the same ranking
        part = oracle.estimate_index_topp(q, k, cu, [n] * hq, [n] * hq, [0.5] * hq, [0.5] * hq, B, 64)
        assert set(part[(h, s)][0]) <= set(iv) and set(part[(h, s)][1]) <= set(is_)
        assert v[part[(h, s)][0] - cu[s]].sum() >= 0.5 * v.sum()


# ---------------------------------------------------------------- P7 RoPE / Theorem 3.1
def test_p7_rope_shift_invariance():
    rng = np.random.default_rng(11)
    d = 128
    for _ in range(20):
        q, k = rng.standard_normal(d), rng.standard_normal(d)
        n, m = rng.integers(0, 524288, size=2)
        t = int(rng.integers(-min(n, m), 524288 - max(n, m)))
        z1 = orope.rope(q, n) @ orope.rope(k, m)
        z2 = orope.rope(q, n + t) @ orope.rope(k, m + t)
        assert abs(z1 - z2) <= 1e-10 * max(1.0, abs(z1))


def test_p7_rope_expectation_matches_eq14():
    """Monte Carlo mean of z at fixed n - m agrees with Eq. 14 within 5 standard errors."""
    rng = np.random.default_rng(12)
    d, ns = 16, 100000
    mu_q, mu_k = rng.standard_normal(d), rng.standard_normal(d)
    Lm = rng.standard_normal((2 * d, 2 * d)) * 0.3
    cov = Lm @ Lm.T + np.eye(2 * d) * 0.2
    x = rng.multivariate_normal(np.concatenate([mu_q, mu_k]), cov, size=ns)
    qs, ks = x[:, :d], x[:, d:]
    C = cov[:d, d:]
    for n, m in ((7, 3), (1000, 996), (40, 0), (300, 260)):
        z = (orope.rope(qs, np.full(ns, n)) * orope.rope(ks, np.full(ns, m))).sum(1)
        se = z.std() / math.sqrt(ns)
        ez = orope.expected_score(n - m, mu_q, mu_k, C)
        assert abs(z.mean() - ez) < 5 * se, (n, m, z.mean(), ez, se)
    # the closed form itself depends on n - m only and is not symmetric in the sign of n - m
    assert abs(orope.expected_score(4, mu_q, mu_k, C) - orope.expected_score(-4, mu_q, mu_k, C)) > 1e-6


# ---------------------------------------------------------------- P8 invariants
def test_p8_score_normalisation_and_index_invariants():
    rng = np.random.default_rng(13)
    n, hq, hkv, d, B = 640, 4, 2, 16, 64
    q = rng.standard_normal((n, hq, d))
    k = rng.standard_normal((n, hkv, d))
    cu = [0, 192, 640]
    vb, sb = [100, 30, 640, 0], [64, 500, 7, 640]
    idx, sc = oracle.estimate_index(q, k, cu, vb, sb, B, 64, return_scores=True)
    for (h, s), (iv, is_) in idx.items():
        a, e = cu[s], cu[s + 1]
        kv, kg = oracle.capacities(vb[h], sb[h], e - a, n, B)
        assert iv.size == kv and is_.size == kg
        assert np.all(np.diff(iv) > 0) and np.all(np.diff(is_) > 0)
        assert iv.size == 0 or (iv.min() >= a and iv.max() < e)
        assert is_.size == 0 or (is_.min() >= 0 and is_.max() < -(-(e - a) // B))
        v, sigma = sc[(h, s)]
        w = min(64, e - a)
        assert abs(v.sum() - w) < 1e-9 and abs(sigma.sum() - w) < 1e-9
    # capacities: single segment gives (min(kv, N), min(ceil(ks/B), N/B))
    assert oracle.capacities(2048, 8192, 131072, 131072, 64) == (2048, 128)
    assert oracle.capacities(64, 64, 1024, 1024, 64) == (64, 1)
    assert oracle.capacities(5000, 10 ** 6, 1024, 1024, 64) == (1024, 16)


def test_estimator_window_matches_plain_softmax():
    """The window probabilities are a plain causal softmax of the last rows (Algorithm 1)."""
    rng = np.random.default_rng(14)
    n, d = 200, 8
    q, k = rng.standard_normal((n, d)), rng.standard_normal((n, d))
    rows, P, lse = oracle.window_probs(q, k, 0, n, 0.5, 64)
    for j, r in enumerate(rows):
        t = torch.softmax(torch.tensor(0.5 * q[r] @ k[: r + 1].T), 0).numpy()
        assert np.abs(P[j, : r + 1] - t).max() < 1e-14 and np.all(P[j, r + 1:] == 0)


# ---------------------------------------------------------------- P9 layout identities
def test_p8_golden_segment_capacities():
    """Per-document budget shares of packed documents (reading of the pages'
    budgets for several documents; values worked out by hand in the fixture):
    a document of L out of N tokens gets ceil(k*L/N) columns and
    ceil(ceil(k*L/N)/64) block-diagonals, clipped to its candidates.  A floor in
    place of a ceiling, L/N inverted or the clip dropped fails a case."""
    with open(os.path.join(GOLDEN, "segment_capacities.json")) as f:
        fx = json.load(f)
    cu, n, B = fx["cu_seqlens"], fx["n_total"], fx["block"]
    assert cu[-1] == n
    for case in fx["cases"]:
        got = [list(oracle.capacities(case["v_budget"], case["s_budget"], cu[s + 1] - cu[s], n, B))
               for s in range(len(cu) - 1)]
        assert got == case["expected"], (case, got)


def test_p9_striped_chunks_merge_to_global_rows():
    rng = np.random.default_rng(15)
    W, B, nbw = 4, 16, 3
    n = W * nbw * B
    hq, hkv, d = 2, 1, 8
    q, do = rng.standard_normal((n, hq, d)), rng.standard_normal((n, hq, d))
    k, v = rng.standard_normal((n, hkv, d)), rng.standard_normal((n, hkv, d))
    idx = rand_index(rng, n, hq, B, kv=10, kg=4)
    pos = np.arange(n)
    Og, Lg = oracle.attn_fwd_dense(q, k, v, pos, pos, [0, n], idx, B)
    Dg = (Og * do).sum(-1).T
    dqg, dkg, dvg = oracle.attn_bwd_dense(q, k, v, do, Lg, Dg, pos, pos, [0, n], idx, B)
    dk_sum = np.zeros_like(k)
    dv_sum = np.zeros_like(v)
    for w in range(W):
        rows = (np.arange(w, n // B, W)[:, None] * B + np.arange(B)).reshape(-1)
        acc_o, acc_l = np.zeros((hq, rows.size, d)), np.full((hq, rows.size), -np.inf)
        for t in range(W):
            u = (w - t) % W
            cols = (np.arange(u, n // B, W)[:, None] * B + np.arange(B)).reshape(-1)
            o, l = oracle.attn_fwd_support(q[rows], k[cols], v[cols], rows, cols, [0, n], idx, B)
            o2, l2 = oracle.attn_fwd_dense(q[rows], k[cols], v[cols], rows, cols, [0, n], idx, B)
            assert np.allclose(o, o2, atol=1e-12) and np.array_equal(np.isneginf(l), np.isneginf(l2))
            acc_o, acc_l = oracle.lse_merge(acc_o, acc_l, o.transpose(1, 0, 2), l)
        assert np.abs(acc_o.transpose(1, 0, 2) - Og[rows]).max() < 1e-12
        fin = np.isfinite(Lg[:, rows])
        assert np.abs(acc_l[fin] - Lg[:, rows][fin]).max() < 1e-12
        D = (acc_o.transpose(1, 0, 2) * do[rows]).sum(-1).T
        dq = np.zeros((rows.size, hq, d))
        for t in range(W):
            u = (w - t) % W
            cols = (np.arange(u, n // B, W)[:, None] * B + np.arange(B)).reshape(-1)
            a, b_, c = oracle.attn_bwd_support(q[rows], k[cols], v[cols], do[rows], acc_l, D, rows,
                                               cols, [0, n], idx, B)
            dq += a
            dk_sum[cols] += b_
            dv_sum[cols] += c
        assert np.abs(dq - dqg[rows]).max() < 1e-12
    assert np.abs(dk_sum - dkg).max() < 1e-12 and np.abs(dv_sum - dvg).max() < 1e-12


def test_p9_packed_documents_equal_documents_alone():
    rng = np.random.default_rng(16)
    B, hq, hkv, d = 16, 2, 1, 8
    cu = [0, 48, 80, 176]
    n = cu[-1]
    q, do = rng.standard_normal((n, hq, d)), rng.standard_normal((n, hq, d))
    k, v = rng.standard_normal((n, hkv, d)), rng.standard_normal((n, hkv, d))
    vb, sb = [40, 20], [64, 30]
    idx = oracle.estimate_index(q, k, cu, vb, sb, B, 16)
    pos = np.arange(n)
    O, L = oracle.attn_fwd_dense(q, k, v, pos, pos, cu, idx, B)
    for s in range(3):
        a, e = cu[s], cu[s + 1]
        sl = slice(a, e)
        # the same document alone, with its share of the budget as the whole budget
        kvs = [oracle.capacities(vb[h], sb[h], e - a, n, B) for h in range(hq)]
        idx1 = oracle.estimate_index(q[sl], k[sl], [0, e - a], [c[0] for c in kvs],
                                     [c[1] * B for c in kvs], B, 16)
        for h in range(hq):
            assert np.array_equal(idx1[(h, 0)][0] + a, idx[(h, s)][0])
            assert np.array_equal(idx1[(h, 0)][1], idx[(h, s)][1])
        p1 = np.arange(e - a)
        O1, L1 = oracle.attn_fwd_dense(q[sl], k[sl], v[sl], p1, p1, [0, e - a], idx1, B)
        assert np.abs(O1 - O[sl]).max() < 1e-12
        fin = np.isfinite(L1)
        assert np.array_equal(fin, np.isfinite(L[:, sl]))
        assert np.abs(L1[fin] - L[:, sl][fin]).max() < 1e-12


# ---------------------------------------------------------------- forms (i) and (ii) agree
def test_support_form_equals_dense_form():
    rng = np.random.default_rng(17)
    B, hq, hkv, d = 16, 4, 2, 8
    cu = [0, 40, 112, 160]
    n = cu[-1]
    q, do = rng.standard_normal((n, hq, d)), rng.standard_normal((n, hq, d))
    k, v = rng.standard_normal((n, hkv, d)), rng.standard_normal((n, hkv, d))
    idx = rand_index(rng, n, hq, B, cu=cu)
    pos = np.arange(n)
    O, L = oracle.attn_fwd_dense(q, k, v, pos, pos, cu, idx, B)
    O2, L2 = oracle.attn_fwd_support(q, k, v, pos, pos, cu, idx, B)
    assert np.array_equal(np.isneginf(L), np.isneginf(L2))
    assert np.abs(O - O2).max() < 1e-12
    fin = np.isfinite(L)
    assert np.abs(L[fin] - L2[fin]).max() < 1e-12
    D = (O * do).sum(-1).T
    g1 = oracle.attn_bwd_dense(q, k, v, do, L, D, pos, pos, cu, idx, B)
    g2 = oracle.attn_bwd_support(q, k, v, do, L, D, pos, pos, cu, idx, B)
    for a, b in zip(g1, g2):
        assert np.abs(a - b).max() < 1e-12


# ---------------------------------------------------------------- P10 accounting
def test_p10_mask_area_formula_equals_count():
    rng = np.random.default_rng(18)
    for cu, B in (([0, 256], 64), ([0, 100, 164, 300], 32), ([0, 1000], 64)):
        n = cu[-1]
        idx = rand_index(rng, n, 3, B, cu=cu)
        pos = np.arange(n)
        assert oracle.mask_area_bruteforce(pos, pos, cu, idx, 3, B) == \
            oracle.mask_area_formula(cu, idx, 3, B)


def test_p10_golden_mask_areas():
    """The cost-model examples: full block S_q*S_k, causal diagonal S_q(S_q+1)/2, and
    the two-sample varlen causal mask of lengths 21 and 11."""
    with open(os.path.join(GOLDEN, "mask_area.json")) as f:
        fx = json.load(f)
    for case in fx["cases"]:
        cu, B = case["cu_seqlens"], case["block"]
        n = cu[-1]
        idx = full_index(n, 1, B, cu) if case["mask"] == "causal" else None
        pos = np.arange(n)
        assert oracle.mask_area_bruteforce(pos, pos, cu, idx, 1, B)[0] == case["area"]
        assert oracle.dense_causal_area(pos, cu) == case["area"]


# ---------------------------------------------------------------- rounding bound of the bf16 backward
def test_bwd_rounding_bound_holds_for_simulated_bf16():
    """A backward that rounds P, dS and O to bf16 (simulated here with torch on the CPU)
    stays inside oracle.bwd_rounding_bounds element by element, and the bound is
    not vacuous (the simulated error reaches a visible fraction of it)."""
    rng = np.random.default_rng(19)
    n, hq, hkv, d, B = 256, 2, 1, 32, 32
    bf = lambda x: torch.tensor(x).to(torch.bfloat16).to(torch.float64).numpy()
    q, do = bf(rng.standard_normal((n, hq, d))), bf(rng.standard_normal((n, hq, d)))
    k, v = bf(rng.standard_normal((n, hkv, d))), bf(rng.standard_normal((n, hkv, d)))
    k[17] *= 6
    pos = np.arange(n)
    idx = rand_index(rng, n, hq, B, kv=20, kg=3)
    O, L = oracle.attn_fwd_dense(q, k, v, pos, pos, [0, n], idx, B)
    D = oracle.bwd_delta(O, do)
    dq, dk, dv = oracle.attn_bwd_dense(q, k, v, do, L, D, pos, pos, [0, n], idx, B)
    bq, bk, bv = oracle.bwd_rounding_bounds(q, k, v, do, O, L, pos, pos, [0, n], idx, B)
    scale = 1 / math.sqrt(d)
    # forward as the GPU does it: P rounded before P V, O stored in bf16
    Ob = np.zeros_like(O)
    for h in range(hq):
        M = oracle.dense_mask(pos, pos, [0, n], idx, h, B)
        S = np.where(M, scale * q[:, h] @ k[:, 0].T, -np.inf)
        A = np.where(M, np.exp(S - np.where(np.isfinite(L[h]), L[h], 0)[:, None]), 0)
        Ob[:, h] = bf(bf(A) @ v[:, 0])
    Dt = (Ob * do).sum(-1).T
    sq, sk, sv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for h in range(hq):
        M = oracle.dense_mask(pos, pos, [0, n], idx, h, B)
        S = np.where(M, scale * q[:, h] @ k[:, 0].T, -np.inf)
        A = np.where(M, np.exp(S - np.where(np.isfinite(L[h]), L[h], 0)[:, None]), 0)
        dS = bf(A * (do[:, h] @ v[:, 0].T - Dt[h][:, None]))
        sq[:, h] = scale * dS @ k[:, 0]
        sk[:, 0] += scale * dS.T @ q[:, h]
        sv[:, 0] += bf(A).T @ do[:, h]
    for sim, ref, b in ((sq, dq, bq), (sk, dk, bk), (sv, dv, bv)):
        err = np.abs(sim - ref)
        assert np.all(err <= 1.01 * b + 1e-12)
        assert (err / (b + 1e-30)).max() > 0.05


# ---------------------------------------------------------------- XAttention block estimator (f4)
from fractions import Fraction

from oracle import xattn as oxa


def test_x1_antidiagonal_sampling_one_hot():
    """Only an anti-diagonal pair of a 16 x 16 cell reaches the cell logit:
    one query row and one key row carry the same unit vector, everything else
    is zero, so z[A, C] is nonzero exactly when (row, key) is the pair
    (16A + u, 16C + 15 - u) of that cell, where it is scale / 16."""
    n, d, S = 64, 8, 16
    for r0, c0, hit in ((17, 30, True), (17, 17, False), (35, 12, True), (35, 3, False),
                        (0, 15, True), (15, 0, True), (20, 20, False), (63, 48, True),
                        (3, 28, True)):  # on an anti-diagonal, but of a cell above the diagonal (X3)
        q = np.zeros((n, d))
        k = np.zeros((n, d))
        q[r0, 3] = 1.0
        k[c0, 3] = 1.0
        z = oxa.antidiag_logits(q, k, 0, n, 0.5, S)
        fin = np.where(np.isfinite(z), z, 0.0)
        A, C = r0 // S, c0 // S
        on_anti = (r0 % S) + (c0 % S) == S - 1
        assert on_anti == hit, (r0, c0)
        expect = np.zeros_like(fin)
        if hit and C <= A:
            expect[A, C] = 0.5 / S
        assert np.array_equal(fin, expect), (r0, c0)


def _uniform_block_scores(nI, cpb=8):
    """Block scores of all-zero logits, worked out with exact fractions: cell
    row A spreads 1/(A+1) over its A+1 causal cells."""
    s = [[Fraction(0)] * nI for _ in range(nI)]
    for A in range(nI * cpb):
        I = A // cpb
        for C in range(A + 1):
            s[I][C // cpb] += Fraction(1, A + 1)
    return s


def test_x2_uniform_scores_closed_form_and_ties():
    """Q = 0: every cell logit is 0.  Block scores equal the exact sums, and
    the selection follows them: with 3 blocks, I = 2 sees J = 0 and J = 1 tie
    exactly (8 * (H_24 - H_16) each); a threshold that one block meets keeps
    J = 0 (lowest index)."""
    n, d = 384, 8
    rng = np.random.default_rng(50)
    q = np.zeros((n, 1, d))
    k = rng.standard_normal((n, 1, d))
    s = oxa.xattn_block_scores(q[:, 0], k[:, 0], 0, n, 0.125)
    exact = _uniform_block_scores(3)
    for I in range(3):
        for J in range(3):
            assert abs(s[I, J] - float(exact[I][J])) < 1e-12, (I, J)
    assert exact[2][0] == exact[2][1]
    for tau, want in ((0.9, {0: [0], 1: [0, 1], 2: [0, 1, 2]}),
                      (0.6, {0: [0], 1: [0], 2: [0, 1]}),
                      (0.3, {0: [0], 1: [0], 2: [0]})):
        idx, sc, cnt = oxa.estimate_index_xattn(q, k, [0, n], threshold=tau, return_scores=True)
        sel = idx[(0, 0)][2][1]
        for I, Js in want.items():
            assert np.nonzero(sel[I])[0].tolist() == Js, (tau, I)
            assert cnt[(0, 0)][I] == len(Js)


def test_x2_cell_logit_is_the_mean():
    """Equal scaled scores x on every sampled pair give z = x (the mean of the
    16 samples, not their sum)."""
    n, d, S = 64, 4, 16
    vec = np.array([1.0, 2.0, -1.0, 0.5])
    q = np.tile(vec, (n, 1))
    k = np.tile(vec, (n, 1))
    z = oxa.antidiag_logits(q, k, 0, n, 0.25, S)
    x = 0.25 * float(vec @ vec)
    fin = np.isfinite(z)
    assert np.allclose(z[fin], x, rtol=0, atol=1e-14)
    assert fin.sum() == (n // S) * (n // S + 1) // 2


def test_x4_block_scores_sum_to_cell_rows():
    """Each cell row's probabilities sum to 1, so a query block's scores sum
    to its cell rows: 8, or 4 for a segment ending half-way through a block."""
    rng = np.random.default_rng(51)
    d = 16
    for L in (512, 576):
        q, k = rng.standard_normal((L, d)) * 2, rng.standard_normal((L, d)) * 2
        s = oxa.xattn_block_scores(q, k, 0, L, 1 / 4)
        rows = np.full(s.shape[0], 8.0)
        if L % 128:
            rows[-1] = (L % 128) / 16
        assert np.abs(s.sum(axis=1) - rows).max() < 1e-12
        assert np.all(np.triu(s, 1) == 0)


def test_x6_threshold_one_is_block_causal_attention():
    """Threshold 1 keeps every key block with a positive score, i.e. every
    J <= I: the mask is plain causal attention, forward and backward equal
    torch's causal SDPA in fp64."""
    rng = np.random.default_rng(52)
    n, hq, hkv, d = 384, 2, 1, 16
    q, k, v, do = (rng.standard_normal((n, h, d)) for h in (hq, hkv, hkv, hq))
    idx = oxa.estimate_index_xattn(q, k, [0, n], threshold=1.0)
    for h in range(hq):
        sel = idx[(h, 0)][2][1]
        assert np.array_equal(sel, np.tril(np.ones_like(sel)))
    pos = np.arange(n)
    O, L = oracle.attn_fwd_dense(q, k, v, pos, pos, [0, n], idx)
    qt = torch.tensor(q).permute(1, 0, 2)[None]
    kt = torch.tensor(k).permute(1, 0, 2)[None].repeat_interleave(hq // hkv, dim=1)
    vt = torch.tensor(v).permute(1, 0, 2)[None].repeat_interleave(hq // hkv, dim=1)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True)
    assert np.abs(O - ref[0].permute(1, 0, 2).numpy()).max() < 1e-12


def test_block_selection_mask_and_forms():
    """A block selection in the index: the mask is causal and the key's block
    selected for the row's block (brute force), and the dense and support
    forms of attention agree on it, with and without Vertical-Slash entries."""
    rng = np.random.default_rng(53)
    B, bb, hq, hkv, d = 16, 32, 2, 1, 8
    cu = [0, 96, 192]
    n = cu[-1]
    q, do = rng.standard_normal((n, hq, d)), rng.standard_normal((n, hq, d))
    k, v = rng.standard_normal((n, hkv, d)), rng.standard_normal((n, hkv, d))
    vs_idx = rand_index(rng, n, hq, B, cu=cu)
    for with_vs in (False, True):
        idx = {}
        for key, (iv, is_) in vs_idx.items():
            L = cu[key[1] + 1] - cu[key[1]]
            nI = -(-L // bb)
            sel = np.tril(rng.random((nI, nI)) < 0.4)
            e = np.zeros(0, np.int64)
            idx[key] = (iv, is_, (bb, sel)) if with_vs else (e, e, (bb, sel))
        pos = np.arange(n)
        for h in range(hq):
            M = oracle.dense_mask(pos, pos, cu, idx, h, B)
            for nn in range(0, n, 7):
                for mm in range(0, n, 5):
                    s = np.searchsorted(cu, nn, side="right") - 1
                    a = cu[s]
                    iv, is_, (_, sel) = idx[(h, s)]
                    same = a <= mm < cu[s + 1]
                    want = same and mm <= nn and (mm in iv or ((nn - a) // B - (mm - a) // B) in is_
                                                 or sel[(nn - a) // bb, (mm - a) // bb])
                    assert M[nn, mm] == want, (with_vs, h, nn, mm)
        O, L = oracle.attn_fwd_dense(q, k, v, pos, pos, cu, idx, B)
        O2, L2 = oracle.attn_fwd_support(q, k, v, pos, pos, cu, idx, B)
        fin = np.isfinite(L)
        assert np.array_equal(fin, np.isfinite(L2)) and np.abs(O - O2).max() < 1e-12
        assert np.abs(L[fin] - L2[fin]).max() < 1e-12
        D = (O * do).sum(-1).T
        g1 = oracle.attn_bwd_dense(q, k, v, do, L, D, pos, pos, cu, idx, B)
        g2 = oracle.attn_bwd_support(q, k, v, do, L, D, pos, pos, cu, idx, B)
        for x, y in zip(g1, g2):
            assert np.abs(x - y).max() < 1e-12


# ---------------------------------------------------------------- MoBA (M1-M5)
from oracle import moba as omb  # noqa: E402


def test_m1_m2_block_means_and_scores_closed_form():
    """Key blocks constant inside a block: each mean is that constant, the
    short last block included (M1), and a query that is a unit vector scores
    each block by that component of its constant (M2)."""
    B, d = 8, 4
    L = 3 * B + 5                       # three whole blocks and a short one
    vals = np.array([[1.0, 0, 0, 0], [0, 2.0, 0, 0], [0, 0, -3.0, 0], [0.5, 0.5, 0.5, 0.5]])
    k = np.concatenate([np.tile(vals[b], (min(B, L - b * B), 1)) for b in range(4)])
    kb = omb.block_means(k, 0, L, B)
    assert np.array_equal(kb, vals)
    q = np.zeros((L, d))
    q[:, 1] = 1.0
    s = omb.gate_scores(q, k, 0, L, B)
    assert np.array_equal(s, np.tile(vals[:, 1], (L, 1)))


def test_m3_m4_selection_property_and_ties():
    """Every row picks its own block and no later one (M3); the earlier blocks
    it picks are min(k - 1, own) of them and none it leaves out scores higher,
    or equal with a lower index (M4); two identical key blocks tie exactly and
    the lower one wins."""
    rng = np.random.default_rng(60)
    B, d, L, topk = 4, 3, 40, 4         # 10 blocks
    q = rng.standard_normal((L, d))
    k = rng.standard_normal((L, d))
    k[12:16] = k[4:8]                   # blocks 1 and 3 identical
    s = omb.gate_scores(q, k, 0, L, B)
    assert np.array_equal(s[:, 1], s[:, 3])
    sel = omb.select_blocks(s, B, topk)
    for r in range(L):
        own = r // B
        assert sel[r, own] and not sel[r, own + 1:].any()
        picked = np.nonzero(sel[r, :own])[0]
        left = np.setdiff1d(np.arange(own), picked)
        assert picked.size == min(topk - 1, own)
        for i in picked:
            for j in left:
                assert s[r, i] > s[r, j] or (s[r, i] == s[r, j] and i < j), (r, i, j)
    # a row that sees blocks 1 and 3 tied at the boundary keeps block 1
    tied = [r for r in range(16, L) if sel[r, 1] != sel[r, 3]]
    assert tied and all(sel[r, 1] and not sel[r, 3] for r in tied)


def test_m5_mask_brute_force_and_forms():
    """The per-row block selection as a mask: m <= n and m's block picked for
    n (brute force over every pair, two segments); the dense and support
    forms of attention agree on it, forward and backward."""
    rng = np.random.default_rng(61)
    B, hq, hkv, d, topk = 16, 2, 1, 8, 2
    cu = [0, 80, 176]
    n = cu[-1]
    q, k, v, do = (rng.standard_normal((n, h, d)) for h in (hq, hkv, hkv, hq))
    idx = omb.estimate_index_moba(q, k, cu, block=B, topk=topk)
    pos = np.arange(n)
    for h in range(hq):
        M = oracle.dense_mask(pos, pos, cu, idx, h, 64)
        ref = np.zeros((n, n), bool)
        for sg in range(2):
            a, e = cu[sg], cu[sg + 1]
            sel = idx[(h, sg)][3][1]
            for r in range(a, e):
                for m in range(a, r + 1):
                    ref[r, m] = sel[r - a, (m - a) // B]
        assert np.array_equal(M, ref), h
    O1, L1 = oracle.attn_fwd_dense(q, k, v, pos, pos, cu, idx)
    O2, L2 = oracle.attn_fwd_support(q, k, v, pos, pos, cu, idx)
    assert np.abs(O1 - O2).max() < 1e-12 and np.abs(L1 - L2).max() < 1e-12
    D = oracle.bwd_delta(O1, do)
    g1 = oracle.attn_bwd_dense(q, k, v, do, L1, D, pos, pos, cu, idx)
    g2 = oracle.attn_bwd_support(q, k, v, do, L1, D, pos, pos, cu, idx)
    for a_, b_ in zip(g1, g2):
        assert np.abs(a_ - b_).max() < 1e-12


def test_m4_enough_blocks_is_causal_attention():
    """top-k at least the number of blocks picks every block up to the own
    one: plain causal attention, equal to torch's causal SDPA in fp64."""
    rng = np.random.default_rng(62)
    n, hq, hkv, d, B = 192, 2, 1, 16, 32
    q, k, v = (rng.standard_normal((n, h, d)) for h in (hq, hkv, hkv))
    idx = omb.estimate_index_moba(q, k, [0, n], block=B, topk=n // B)
    for h in range(hq):
        sel = idx[(h, 0)][3][1]
        own = np.arange(n) // B
        assert np.array_equal(sel, np.arange(n // B)[None, :] <= own[:, None])
    pos = np.arange(n)
    O, _ = oracle.attn_fwd_dense(q, k, v, pos, pos, [0, n], idx)
    qt = torch.tensor(q).permute(1, 0, 2)[None]
    kt = torch.tensor(k).permute(1, 0, 2)[None].repeat_interleave(hq // hkv, dim=1)
    vt = torch.tensor(v).permute(1, 0, 2)[None].repeat_interleave(hq // hkv, dim=1)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True)
    assert np.abs(O - ref[0].permute(1, 0, 2).numpy()).max() < 1e-12
