"""Seeded synthetic inputs for Vertical-Slash sparse attention.

This module only draws random tensors and lays them out.  It holds none of the
attention method's arithmetic (no scores, softmax, selection or masks), so the
CPU oracle and the GPU path can both consume its output without sharing code.

Recipe (one call per workload):
  1. ``torch.Generator('cpu').manual_seed(seed)``  (default 1000 + workload id);
  2. in this order draw fp32 ``randn``: Q [1,N,Hq,d], K [1,N,Hkv,d],
     V [1,N,Hkv,d], dO [1,N,Hq,d];
  3. outlier key positions: ``randperm(N)[:n_out]`` (n_out = round(frac*N),
     at least 1 when frac > 0);
  4. packed documents: ``randperm(N/64 - 1)[:n_docs-1] + 1`` sorted, times 64,
     are the interior cut points; then per-Q-head budgets with ``randint``;
  5. outlier K rows (every KV head) are multiplied by the outlier factor;
  6. rotary position embedding (rotate-half, theta_i = base^(-2i/d)) applied
     in fp64 at the global positions 0..N-1 to Q and K;
  7. everything is rounded to the workload dtype.

Outlier keys with a large norm stand in for the "vertical" columns and RoPE for
the relative-position "slash" structure that MTraining (arXiv 2510.18830,
§3.2, Theorem 3.1) attributes the Vertical-Slash pattern to.  With independent
zero-mean Q and K the expected slash structure is flat; these inputs exercise
shapes, masks and kernels, not model behaviour.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional

import torch

BLOCK = 64

# The five workloads: shapes, dtype, budgets (tokens) and input recipe.
WORKLOADS = {
    1: dict(name="tiny-fp32-n1024", dtype="f32", h_q=1, h_kv=1, d=64, n=1024,
            n_out=4, out_factor=8.0, v_budget=64, s_budget=64),
    2: dict(name="qwen2.5-3b-layer-n32k", dtype="bf16", h_q=16, h_kv=2, d=128, n=32768,
            out_frac=0.001, out_factor=6.0, v_budget=1024, s_budget=4096),
    3: dict(name="qwen2.5-3b-layer-n128k", dtype="bf16", h_q=16, h_kv=2, d=128, n=131072,
            out_frac=0.001, out_factor=6.0, v_budget=2048, s_budget=8192),
    4: dict(name="striped-ring-worker-n512k", dtype="bf16", h_q=16, h_kv=2, d=128, n=524288,
            out_frac=0.001, out_factor=6.0, v_budget=4096, s_budget=20480,
            stripe_world=32, stripe_rank=0),
    5: dict(name="packed-docs-n256k", dtype="bf16", h_q=16, h_kv=2, d=128, n=262144,
            out_frac=0.001, out_factor=6.0, n_docs=8,
            v_budget_range=(512, 4096), s_budget_range=(2048, 16384)),
}


@dataclasses.dataclass
class Problem:
    """One seeded problem instance (CPU tensors, layout [batch, token, head, dim])."""
    wid: int
    name: str
    dtype: str                 # "f32" or "bf16": the dtype q/k/v/do are rounded to
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    do: torch.Tensor
    h_q: int
    h_kv: int
    d: int
    n: int
    block: int
    cu_seqlens: List[int]      # segment boundaries in tokens, [0, ..., n]
    v_budget: List[int]        # per Q head, tokens
    s_budget: List[int]        # per Q head, tokens
    outliers: torch.Tensor     # int64 key positions that were scaled
    stripe_world: int = 1
    stripe_rank: int = 0
    seed: int = 0

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16


def rope_rotate_half(x: torch.Tensor, positions: torch.Tensor, base: float = 10000.0,
                     chunk: int = 8192, dtype: Optional[str] = None) -> torch.Tensor:
    """Rotary embedding (rotate-half pairing of dim i with i + d/2), fp64 math.

    x: [1, N, H, d] float tensor; positions: [N] int64.  Returns an fp64
    tensor, or, with ``dtype``, the fp64 result rounded chunk by chunk to that
    dtype (the same values as rounding the whole fp64 tensor afterwards).
    """
    d = x.shape[-1]
    half = d // 2
    inv = base ** (-2.0 * torch.arange(half, dtype=torch.float64) / d)
    out_dtype = torch.float64 if dtype is None else (torch.float32 if dtype == "f32" else torch.bfloat16)
    out = torch.empty(x.shape, dtype=out_dtype)
    for s in range(0, x.shape[1], chunk):
        e = min(x.shape[1], s + chunk)
        ang = positions[s:e].to(torch.float64)[:, None] * inv[None, :]      # [c, half]
        c = torch.cos(ang)[None, :, None, :]
        sn = torch.sin(ang)[None, :, None, :]
        xs = x[:, s:e].to(torch.float64)
        lo, hi = xs[..., :half], xs[..., half:]
        r = torch.cat((lo * c - hi * sn, hi * c + lo * sn), dim=-1)
        out[:, s:e] = r if dtype is None else _round(r, dtype)
    return out


def _round(x64: torch.Tensor, dtype: str) -> torch.Tensor:
    if dtype == "f32":
        return x64.to(torch.float32)
    return x64.to(torch.float32).to(torch.bfloat16)


def make_problem(wid: int, n: Optional[int] = None, seed: Optional[int] = None,
                 h_q: Optional[int] = None, h_kv: Optional[int] = None, d: Optional[int] = None,
                 v_budget=None, s_budget=None, dtype: Optional[str] = None,
                 n_docs: Optional[int] = None, out_frac: Optional[float] = None,
                 stripe_world: Optional[int] = None) -> Problem:
    """Draw workload ``wid`` (1..5), optionally at a reduced size.

    Overrides keep the recipe and change only the named quantity.  Budgets are
    tokens, one value for every head or one per Q head.
    """
    w = dict(WORKLOADS[wid])
    n = n if n is not None else w["n"]
    h_q = h_q if h_q is not None else w["h_q"]
    h_kv = h_kv if h_kv is not None else w["h_kv"]
    d = d if d is not None else w["d"]
    dtype = dtype if dtype is not None else w["dtype"]
    seed = seed if seed is not None else 1000 + wid
    assert n % BLOCK == 0 and h_q % h_kv == 0
    g = torch.Generator("cpu").manual_seed(seed)
    q = torch.randn((1, n, h_q, d), generator=g, dtype=torch.float32)
    k = torch.randn((1, n, h_kv, d), generator=g, dtype=torch.float32)
    v = torch.randn((1, n, h_kv, d), generator=g, dtype=torch.float32)
    do = torch.randn((1, n, h_q, d), generator=g, dtype=torch.float32)
    if "n_out" in w and out_frac is None:
        n_out = w["n_out"] if n == w["n"] else max(1, round(w["n_out"] * n / w["n"]))
    else:
        frac = out_frac if out_frac is not None else w.get("out_frac", 0.0)
        n_out = max(1, round(frac * n)) if frac > 0 else 0
    outliers = torch.randperm(n, generator=g)[:n_out].sort().values
    cu = [0, n]
    docs = n_docs if n_docs is not None else w.get("n_docs", 1)
    if docs > 1:
        nb = n // BLOCK
        assert nb >= docs
        cuts = (torch.randperm(nb - 1, generator=g)[:docs - 1] + 1).sort().values * BLOCK
        cu = [0] + [int(c) for c in cuts] + [n]
    if v_budget is None and "v_budget_range" in w:
        lo, hi = w["v_budget_range"]
        vb = [int(x) for x in torch.randint(lo, hi + 1, (h_q,), generator=g)]
        lo, hi = w["s_budget_range"]
        sb = [int(x) for x in torch.randint(lo, hi + 1, (h_q,), generator=g)]
    else:
        vb = v_budget if v_budget is not None else w["v_budget"]
        sb = s_budget if s_budget is not None else w["s_budget"]
        vb = list(vb) if isinstance(vb, (list, tuple)) else [int(vb)] * h_q
        sb = list(sb) if isinstance(sb, (list, tuple)) else [int(sb)] * h_q
    if n_out:
        k[:, outliers] *= w["out_factor"]
    pos = torch.arange(n, dtype=torch.int64)
    q = rope_rotate_half(q, pos, dtype=dtype)
    k = rope_rotate_half(k, pos, dtype=dtype)
    # fp32 -> fp64 is exact, so V and dO round straight from fp32
    v = _round(v, dtype)
    do = _round(do, dtype)
    sw = stripe_world if stripe_world is not None else w.get("stripe_world", 1)
    return Problem(wid=wid, name=w["name"], dtype=dtype, q=q, k=k, v=v, do=do, h_q=h_q,
                   h_kv=h_kv, d=d, n=n, block=BLOCK, cu_seqlens=cu, v_budget=vb,
                   s_budget=sb, outliers=outliers, stripe_world=sw,
                   stripe_rank=w.get("stripe_rank", 0), seed=seed)


def stripe_positions(n_global: int, world: int, rank: int, block: int = BLOCK) -> torch.Tensor:
    """Global token positions held by ``rank`` under block striping.

    Rank r holds global blocks r, r + world, r + 2*world, ... in that order
    (64-token stripes, MTraining arXiv 2510.18830 §4.2 (ii)).
    """
    nb = n_global // block
    blocks = torch.arange(rank, nb, world, dtype=torch.int64)
    return (blocks[:, None] * block + torch.arange(block, dtype=torch.int64)[None, :]).reshape(-1)


def stripe_rows(x: torch.Tensor, world: int, rank: int, block: int = BLOCK) -> torch.Tensor:
    """Rows of x ([1, N, H, d]) that block-striped rank ``rank`` holds, contiguous."""
    idx = stripe_positions(x.shape[1], world, rank, block)
    return x[:, idx].contiguous()
