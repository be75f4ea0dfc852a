"""Oracle, part 4: RoPE and the relative-position property (test infrastructure only).

MTraining (arXiv 2510.18830) §3.2 Theorem 3.1 and the paper note's Appendix B.2:
with RoPE the score z[n,m] = RoPE(q, n) . RoPE(k, m) equals q W_(n-m) k^T, so it
depends on n and m only through n - m, and its expectation is

  E[z] = sum_i phi_i (mu_q^i mu_k^i + C[i, i])
       + sum_i psi_i (mu_q^i mu_k^p(i) + C[i, p(i)]),

phi_i = cos((n-m) theta_(i mod d/2)), psi_i = (-1)^[i >= d/2] sin((n-m) theta_(i mod d/2)),
p(i) = (i + d/2) mod d (the rotate-half partner; the printed index is garbled
and the appendix's expansion fixes it), theta_j = base^(-2j/d).
"""
from __future__ import annotations

import numpy as np


def rope(x, pos, base=10000.0):
    """Rotate-half RoPE of rows x [..., d] at positions pos [...] (float64)."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    half = d // 2
    theta = base ** (-2.0 * np.arange(half) / d)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * theta
    c, s = np.cos(ang), np.sin(ang)
    lo, hi = x[..., :half], x[..., half:]
    return np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1)


def expected_score(delta, mu_q, mu_k, cross_cov, base=10000.0):
    """Eq. 14: E[z] at relative position delta for moments (mu_q, mu_k, C[i, j] = cov(q_i, k_j))."""
    mu_q = np.asarray(mu_q, np.float64)
    mu_k = np.asarray(mu_k, np.float64)
    C = np.asarray(cross_cov, np.float64)
    d = mu_q.shape[0]
    half = d // 2
    i = np.arange(d)
    theta = base ** (-2.0 * (i % half) / d)
    phi = np.cos(delta * theta)
    psi = np.where(i >= half, -1.0, 1.0) * np.sin(delta * theta)
    p = (i + half) % d
    return float((phi * (mu_q * mu_k + C[i, i])).sum() + (psi * (mu_q * mu_k[p] + C[i, p])).sum())
