"""Shared helpers for the GPU parity tests: seeded problems, oracle runs, comparisons.

Inputs come from the seeded generator (``workloads``); expected values come
from the CPU oracle only.  The oracle's index is handed to the GPU attention
calls, so attention parity does not depend on the estimator's near-ties.
"""
from __future__ import annotations

import math
import sys
import time

import numpy as np
import torch

import oracle
import workloads


def log(msg):
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


def np64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to(torch.float64).cpu().numpy()


def oracle_index(prob: workloads.Problem, last_q=64):
    """Oracle index {(h, seg): (iv, is)} for batch row 0 (float64 estimator)."""
    return oracle.estimate_index(np64(prob.q[0]), np64(prob.k[0]), prob.cu_seqlens, prob.v_budget,
                                 prob.s_budget, prob.block, last_q, return_scores=True)


def lists_for_gpu(index, h_q, n_seg):
    """Oracle index -> list order of the C ABI (l = h * n_seg + s, batch 1)."""
    return [(index[(h, s)][0].tolist(), index[(h, s)][1].tolist())
            for h in range(h_q) for s in range(n_seg)]


def bf16_tol(ref: np.ndarray, got: np.ndarray):
    """(max-abs, relative L2) of got vs ref."""
    err = np.abs(got - ref)
    rel = np.linalg.norm((got - ref).ravel()) / max(np.linalg.norm(ref.ravel()), 1e-30)
    return float(err.max(initial=0.0)), float(rel)


def _bf16_half_ulp(x):
    """Half the spacing of bfloat16 numbers at |x| (the largest output rounding error)."""
    a = np.abs(np.asarray(x, np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, 2.0 ** (e - 8), 0.0)


def check_close(name, ref, got, dtype, kind="out", bound=None):
    """Compare got with ref; returns an error string or None.

    fp32: max-abs <= 1e-4.  bf16 outputs (O, LSE): max-abs <= 2e-2; for O
    (kind "o") the log splits the error into the output's own bf16 rounding
    and the rest.  bf16 gradients: relative L2 <= 1e-2 and, element by
    element, within twice the first-order bf16 rounding bound of the backward
    (oracle.bwd_rounding_bounds).  The log also gives rms(ref) and the ratio of
    the max-abs error to 2e-2 * max(1, rms(ref)): a backward that rounds P and
    dS to bf16 before its products has errors of the size |dS| |K| u, far
    above that bar where a row's probability sits on large-norm keys (the
    bound's maximum is printed beside it).
    """
    ref = np.asarray(ref, np.float64)
    got = np.asarray(got, np.float64)
    if ref.shape != got.shape:
        return f"{name}: shape {got.shape} != {ref.shape}"
    fin_r = np.isfinite(ref)
    fin_g = np.isfinite(got)
    if not np.array_equal(fin_r, fin_g):
        return f"{name}: finite pattern differs ({int((fin_r != fin_g).sum())} entries)"
    if not np.array_equal(ref[~fin_r], got[~fin_g]):
        return f"{name}: infinities differ"
    r, g = ref[fin_r], got[fin_g]
    mx, rel = bf16_tol(r, g)
    rms = float(np.sqrt(np.mean(r * r))) if r.size else 0.0
    extra = ""
    if bound is not None:
        b = np.asarray(bound, np.float64)[fin_r]
        ratio = float((np.abs(g - r) / (b + 1e-30)).max(initial=0.0))
        extra = f" err/bound {ratio:.3f} (bound max {float(b.max(initial=0.0)):.3e})"
    if dtype == "bf16" and kind == "grad":
        q19 = mx / (2e-2 * max(1.0, rms))
        extra += f" rms(ref) {rms:.3e} max-abs/(2e-2*max(1,rms)) {q19:.2f}"
    if dtype == "bf16" and kind == "o" and r.size:
        # the output is stored in bf16: its own rounding is up to half a bf16 spacing
        rb = torch.tensor(r).to(torch.bfloat16).to(torch.float64).numpy()
        extra += (f" (vs bf16-rounded ref {float(np.abs(g - rb).max()):.3e},"
                  f" half-ulp at the worst element {float(_bf16_half_ulp(r)[np.argmax(np.abs(g - r))]):.3e})")
    log(f"  {name}: max-abs {mx:.3e} rel-L2 {rel:.3e}{extra} (n={r.size})")
    if dtype == "f32":
        return None if mx <= 1e-4 else f"{name}: max-abs {mx}"
    if kind in ("out", "o"):
        return None if mx <= 2e-2 else f"{name}: max-abs {mx}"
    if rel > 1e-2:
        return f"{name}: rel-L2 {rel}"
    if bound is not None:
        bad = np.abs(g - r) > 2.0 * b + 1e-6
        if bad.any():
            return f"{name}: {int(bad.sum())} entries beyond 2x rounding bound (worst ratio {ratio:.2f})"
    return None


def assert_close(name, ref, got, dtype, kind="out", bound=None):
    err = check_close(name, ref, got, dtype, kind, bound)
    assert err is None, err


def index_parity(name, o_index, o_scores, g_lists, g_vscore, g_sscore, prob, rel_tie=1e-5):
    """Estimator parity.

    1. scores: GPU fp32 vertical / slash scores against the oracle's fp64 ones;
    2. selection: each GPU list is exactly the top-k of the GPU's own scores
       (ties to the lowest index) — the integer decision in the kernel's
       precision, checked with a plain stable sort;
    3. sets: each GPU list equals the oracle's; a difference is accepted only
       as certified near-ties (oracle scores of every swapped element within
       rel_tie of the k-th score) and is reported.
    Returns the number of near-tie swaps.
    """
    n_seg = len(prob.cu_seqlens) - 1
    swaps = 0
    vmax = 0.0
    for h in range(prob.h_q):
        for s in range(n_seg):
            a, e = prob.cu_seqlens[s], prob.cu_seqlens[s + 1]
            l = h * n_seg + s
            ov, osg = o_scores[(h, s)]
            gv = g_vscore[h, a:e].astype(np.float64)
            gs = g_sscore[h, a // 64: e // 64].astype(np.float64)
            vmax = max(vmax, float(np.abs(gv - ov).max() / max(ov.max(), 1e-30)))
            assert np.abs(gv - ov).max() <= 1e-3 * max(ov.max(), 1e-30) + 1e-6, (name, h, s, "v")
            assert np.abs(gs - osg).max() <= 1e-3 * max(osg.max(), 1e-30) + 1e-6, (name, h, s, "sigma")
            gvl = np.asarray(g_lists[l][0])
            gsl = np.asarray(g_lists[l][1])
            for kind, glist, gsc, olist, osc, off in (("v", gvl, g_vscore[h, a:e], o_index[(h, s)][0], ov, a),
                                                      ("s", gsl, g_sscore[h, a // 64:e // 64], o_index[(h, s)][1], osg, 0)):
                k = olist.size
                assert glist.size == k, (name, kind, h, s, glist.size, k)
                assert np.all(np.diff(glist) > 0), (name, kind, "not ascending")
                # selection in the kernel's precision
                sc32 = np.asarray(gsc, np.float32)
                order = np.lexsort((np.arange(sc32.size), -sc32.astype(np.float64)))
                assert np.array_equal(np.sort(order[:k]) + off, glist), (name, kind, h, s, "not top-k of own scores")
                if not np.array_equal(glist, olist):
                    extra = np.setdiff1d(glist, olist) - off
                    miss = np.setdiff1d(olist, glist) - off
                    kth = np.sort(osc)[::-1][k - 1]
                    tol = rel_tie * max(kth, 1e-30)
                    assert np.all(np.abs(osc[extra] - kth) <= tol) and np.all(np.abs(osc[miss] - kth) <= tol), \
                        (name, kind, h, s, "non-tie mismatch", extra[:5], miss[:5])
                    swaps += extra.size
    log(f"  {name}: index sets match oracle, near-tie swaps={swaps}, max rel score err={vmax:.2e}")
    return swaps


# XAttention block selection: the device scores are fp32 sums of at most 64
# cell probabilities, each an exp2 of a difference of fp32 log-sum-exps of
# dot products accumulated in fp32 over 16 x d terms (relative error a few
# 2^-20 in practice); the bar is 1e-4 * (1 + s), s <= 8 the block's cell rows.
XA_SCORE_RTOL = 1e-4


def xattn_count_int(scores_f32, t):
    """The XAttention selection count in the device's integer arithmetic,
    recomputed from the device's fp32 scores of one query block: masses
    rint(s * 2^50), target ceil(rint(t * 2^24) * total / 2^24), ties to the
    lowest key block.  Returns (count, key blocks in selection order)."""
    tc = np.float32(t)
    tc = np.float32(min(tc, np.float32(1.0))) if tc > 0 else np.float32(0.0)
    tq = int(np.rint(np.float64(tc) * 2.0 ** 24))
    m = np.rint(np.asarray(scores_f32, np.float32).astype(np.float64) * 2.0 ** 50).astype(np.int64)
    order = np.lexsort((np.arange(m.size), -m))
    total = int(m.sum())
    if tq == 0 or total == 0:
        return 0, order
    need = -(-(tq * total) // (1 << 24))
    cum = np.cumsum(m[order])
    return min(int(np.searchsorted(cum, need, side="left")) + 1, m.size), order


def check_xattn_row(tag, so, sg, got_bits, cnt_dev, ko, thr):
    """One query block I of a head: so = the oracle's fp64 scores of key
    blocks 0..I, sg = the device's fp32 scores, got_bits = the device's
    bitmap row (bool, all key blocks), cnt_dev its count, ko the oracle's
    count.  Asserts the scores within XA_SCORE_RTOL, the device's count and
    bitmap equal to the integer decision on its own scores, and the selection
    equal to the oracle's except at a certified boundary flip or near tie.
    Returns (relative score error, flips, swaps)."""
    so = np.asarray(so, np.float64)
    err = np.abs(np.asarray(sg, np.float64) - so)
    assert np.all(err <= XA_SCORE_RTOL * (1 + so)), (tag, float(err.max()))
    kk, order = xattn_count_int(sg, thr)
    assert cnt_dev == kk, (tag, int(cnt_dev), kk)
    want = np.zeros(got_bits.size, bool)
    want[order[:kk]] = True
    assert np.array_equal(got_bits, want), (tag, "bitmap")
    flips = swaps = 0
    if kk != ko:
        srt = np.sort(so)[::-1]
        cum = np.concatenate(([0.0], np.cumsum(srt)))
        tot = cum[-1]
        delta = 2 * err.sum() + 2.0 ** -24 * tot + 1e-12
        tc = min(max(thr, 0.0), 1.0)
        assert cum[kk] >= tc * tot - delta, (tag, kk, ko)
        assert kk == 0 or cum[kk - 1] < tc * tot + delta, (tag, kk, ko)
        flips = 1
    ref = np.sort(np.lexsort((np.arange(so.size), -so))[:kk])
    got = np.nonzero(got_bits)[0]
    if not np.array_equal(ref, got):
        kth = np.sort(so)[::-1][kk - 1]
        diff = np.setxor1d(ref, got)
        assert np.all(np.abs(so[diff] - kth) <= 2 * XA_SCORE_RTOL * (1 + kth)), (tag, "non-tie mismatch")
        swaps = diff.size // 2
    return float((err / (1 + so)).max(initial=0.0)), flips, swaps, ref


def pack_block_selection(sels, nI):
    """Host bitmap rows of block selections sels[r] [nI, nI] (bool), one per
    (batch, Q head) in order: bit J % 32 of word J // 32 of row r * nI + I."""
    words = (nI + 31) // 32
    out = np.zeros((len(sels) * nI, words), np.uint32)
    for r, sel in enumerate(sels):
        I, J = np.nonzero(np.asarray(sel, bool))
        np.bitwise_or.at(out, (r * nI + I, J // 32), (np.uint32(1) << (J % 32).astype(np.uint32)))
    return torch.from_numpy(out.view(np.int32))
