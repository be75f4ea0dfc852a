"""Vertical-Slash dynamic sparse attention on MI355X (gfx950): Python binding.

Thin wrapper over the C ABI of ``include/vs.h`` (libvs.so, hand-written HIP
kernels).  PyTorch provides device memory and the stream; every step of the
method runs in the library's kernels.  There is no CPU fallback: if the
library is not built, the calls raise.

Entry points (same names as the C ABI):
  * ``estimate_index``   — online Vertical-Slash index (MTraining paper note,
    Algorithm 1; MTraining arXiv 2510.18830 §4.1);
  * ``estimate_index_topp`` — the same with top-p budgets (Algorithm 1 topp);
  * ``sparse_attn_fwd``  — sparse attention forward with LSE;
  * ``sparse_attn_bwd``  — dQ, dK, dV over the same support;
  * ``sparse_attn_bwd_noalloc`` — the same with the library's fixed per-GPU
    workspace (for callers that cannot allocate);
  * ``lse_merge``        — merge_out_and_lse of Algorithm 2;
  * ``attn_bwd_delta``   — the row term rowsum(dO * O) of Eq. 1.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import List, Optional, Sequence, Tuple

import torch

from . import _abi
from ._abi import VsError

BLOCK = 64
__all__ = ["VsIndexT", "index_capacity", "estimate_index", "estimate_index_topp",
           "estimate_index_xattn", "estimate_index_moba", "sparse_attn_fwd",
           "sparse_attn_bwd", "sparse_attn_bwd_noalloc",
           "attn_bwd_delta", "lse_merge", "VsError", "BLOCK"]


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return _abi.VS_BF16
    if t.dtype == torch.float32:
        return _abi.VS_F32
    raise ValueError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _small_to_dev(values, dtype, dev: torch.device) -> torch.Tensor:
    """A short host list on the device, staged in pinned memory and copied
    asynchronously on the current stream (a copy from pageable memory would
    first wait for the stream's earlier work)."""
    return torch.tensor(values, dtype=dtype).pin_memory().to(dev, non_blocking=True)


def _need(t: torch.Tensor, name: str, dtype=None, dev=None, strided=False):
    """Checks a tensor argument.  strided: a [batch, token, head, d] view whose
    last dimension is contiguous is accepted (its strides go to the library);
    otherwise the tensor must be contiguous."""
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if strided:
        if t.dim() != 4 or t.stride(3) != 1:
            raise ValueError(f"{name} must be [batch, token, head, d] with d contiguous")
    elif not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if dev is not None and t.device != dev:
        raise ValueError(f"{name} is on {t.device}, expected {dev}")


def _strides(t: Optional[torch.Tensor]):
    return (0, 0, 0) if t is None else tuple(int(x) for x in t.stride()[:3])


class _Problem:
    """A vs_problem plus the host arrays it points to (kept alive).

    stripe = (W, q_rank, k_rank) with k_rank an int or "all" (K/V hold every
    rank's chunk, chunk u after chunk u-1).  Strides are taken from the
    tensors given (q, k, v, o, do); absent ones are contiguous."""

    def __init__(self, batch, h_q, h_kv, d, n_q, n_k, dtype_code, cu_seqlens, stripe, scale,
                 q=None, k=None, v=None, o=None, do=None):
        W, qr, kr = stripe if stripe is not None else (1, 0, 0)
        if kr == "all":
            kr = _abi.VS_ALL_CHUNKS
        n_global = n_q * W
        cu = list(cu_seqlens) if cu_seqlens is not None else [0, n_global]
        self.cu = (ctypes.c_int32 * len(cu))(*[int(x) for x in cu])
        st = [_abi.i64x3(*_strides(t)) for t in (q, k, v, o, do)]
        self.s = _abi.VsProblem(batch, h_q, h_kv, d, n_q, n_k, BLOCK, dtype_code,
                                float(scale) if scale else 0.0, len(cu) - 1,
                                ctypes.cast(self.cu, _abi.i32p), int(W), int(qr), int(kr), *st)
        self.n_seg = len(cu) - 1

    @property
    def ref(self):
        return ctypes.byref(self.s)


@dataclass
class VsIndexT:
    """The Vertical-Slash index on the device (CSR per (batch, Q head, segment)).

    blk_mask (optional): a block selection instead of the lists, one bit per
    (batch, Q head, query block, key block) of blk_size tokens, rows of
    ceil(nI / 32) int32 words (the layout estimate_index_xattn writes).
    row_mask (optional): a per-row block selection, one int32 word per
    (batch, Q head, row) whose bit J marks key block J of row_blk tokens (the
    layout estimate_index_moba writes)."""
    v_ptr: torch.Tensor
    v_idx: torch.Tensor
    s_ptr: torch.Tensor
    s_idx: torch.Tensor
    v_cap_max: int
    s_cap_max: int
    blk_mask: Optional[torch.Tensor] = None
    blk_size: int = 0
    row_mask: Optional[torch.Tensor] = None
    row_blk: int = 0

    def struct(self) -> _abi.VsIndex:
        return _abi.VsIndex(self.v_ptr.data_ptr(), self.v_idx.data_ptr(), self.s_ptr.data_ptr(),
                            self.s_idx.data_ptr(), self.v_cap_max, self.s_cap_max,
                            None if self.blk_mask is None else self.blk_mask.data_ptr(),
                            self.blk_size,
                            None if self.row_mask is None else self.row_mask.data_ptr(),
                            self.row_blk)

    def block_selection(self, n: int):
        """Host copy of a block selection as bool [B*Hq, nI, nI] (n tokens per row)."""
        nI = -(-n // self.blk_size)
        w = self.blk_mask.cpu().view(-1, nI, -(-nI // 32)).to(torch.int64) & 0xFFFFFFFF
        bits = (w.unsqueeze(-1) >> torch.arange(32)) & 1
        return bits.flatten(-2)[..., :nI].bool()

    def lists(self):
        """Host copy: list number -> (verticals, block-diagonals) as int tensors."""
        vp, vi = self.v_ptr.cpu(), self.v_idx.cpu()
        sp, si = self.s_ptr.cpu(), self.s_idx.cpu()
        return [(vi[vp[l]:vp[l + 1]], si[sp[l]:sp[l + 1]]) for l in range(vp.numel() - 1)]


_ws_cache = {}


def _workspace(dev: torch.device, nbytes: int) -> torch.Tensor:
    buf = _ws_cache.get(dev)
    if buf is None or buf.numel() < nbytes:
        buf = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
        _ws_cache[dev] = buf
    return buf


def index_capacity(batch: int, h_q: int, h_kv: int, d: int, n: int, v_budget: Sequence[int],
                   s_budget: Sequence[int], cu_seqlens=None, dtype_code: int = _abi.VS_BF16):
    """Host CSR offsets for budgets (tokens per Q head); returns (v_ptr, s_ptr, v_max, s_max)."""
    P = _Problem(batch, h_q, h_kv, d, n, n, dtype_code, cu_seqlens, None, None)
    nl = batch * h_q * P.n_seg
    vp = (ctypes.c_int32 * (nl + 1))()
    sp = (ctypes.c_int32 * (nl + 1))()
    vb = (ctypes.c_int32 * h_q)(*[int(x) for x in v_budget])
    sb = (ctypes.c_int32 * h_q)(*[int(x) for x in s_budget])
    vm, sm = ctypes.c_int32(), ctypes.c_int32()
    _abi.check(_abi.lib().vs_index_capacity(P.ref, vb, sb, vp, sp, ctypes.byref(vm), ctypes.byref(sm)))
    return list(vp), list(sp), vm.value, sm.value


def estimate_index(q: torch.Tensor, k: torch.Tensor, v_budget: Sequence[int],
                   s_budget: Sequence[int], cu_seqlens=None, return_scores: bool = False):
    """Online Vertical-Slash index for q [B, N, Hq, d], k [B, N, Hkv, d] (contiguous layout).

    Budgets are tokens per Q head.  Returns a VsIndexT (and, with
    return_scores, the vertical scores [B, Hq, N] and slash scores [B, Hq, N/64]).
    """
    dev = q.device
    _need(q, "q", dev=dev, strided=True)
    _need(k, "k", q.dtype, dev, strided=True)
    B, N, Hq, d = q.shape
    Hkv = k.shape[2]
    dc = _dtype_code(q)
    vp, sp, vm, sm = index_capacity(B, Hq, Hkv, d, N, v_budget, s_budget, cu_seqlens, dc)
    P = _Problem(B, Hq, Hkv, d, N, N, dc, cu_seqlens, None, None, q=q, k=k)
    v_ptr = _small_to_dev(vp, torch.int32, dev)
    s_ptr = _small_to_dev(sp, torch.int32, dev)
    v_idx = torch.empty(max(vp[-1], 1), dtype=torch.int32, device=dev)
    s_idx = torch.empty(max(sp[-1], 1), dtype=torch.int32, device=dev)
    v_score = torch.empty((B, Hq, N), dtype=torch.float32, device=dev) if return_scores else None
    s_score = torch.empty((B, Hq, N // BLOCK), dtype=torch.float32, device=dev) if return_scores else None
    L = _abi.lib()
    nb = ctypes.c_size_t()
    _abi.check(L.vs_workspace_size(P.ref, 0, None, ctypes.byref(nb)))
    ws = _workspace(dev, nb.value)
    _abi.check(L.vs_estimate_index(P.ref, _ptr(q), _ptr(k), 0, _ptr(v_ptr), _ptr(v_idx), _ptr(s_ptr),
                                   _ptr(s_idx), _ptr(v_score), _ptr(s_score), _ptr(ws), ws.numel(),
                                   _stream(dev)))
    idx = VsIndexT(v_ptr, v_idx, s_ptr, s_idx, vm, sm)
    return (idx, v_score, s_score) if return_scores else idx


def estimate_index_topp(q: torch.Tensor, k: torch.Tensor, v_cap: Sequence[int], s_cap: Sequence[int],
                        p_v: Sequence[float], p_s: Sequence[float], cu_seqlens=None,
                        return_scores: bool = False):
    """Online Vertical-Slash index with top-p budgets: per (Q head, segment) the
    fewest top verticals / block-diagonals holding a share p_v[h] / p_s[h] of the
    window mass, at most the capacities of the token budgets v_cap / s_cap.

    Returns (VsIndexT, counts [B*Hq*n_seg, 2] int32 = (k_v, k_s) per list) and,
    with return_scores, also the vertical and slash scores.  Unused capacity is
    padded with -1.
    """
    dev = q.device
    _need(q, "q", dev=dev, strided=True)
    _need(k, "k", q.dtype, dev, strided=True)
    B, N, Hq, d = q.shape
    Hkv = k.shape[2]
    if len(p_v) != Hq or len(p_s) != Hq:
        raise ValueError(f"p_v and p_s need {Hq} entries")
    dc = _dtype_code(q)
    vp, sp, vm, sm = index_capacity(B, Hq, Hkv, d, N, v_cap, s_cap, cu_seqlens, dc)
    P = _Problem(B, Hq, Hkv, d, N, N, dc, cu_seqlens, None, None, q=q, k=k)
    v_ptr = _small_to_dev(vp, torch.int32, dev)
    s_ptr = _small_to_dev(sp, torch.int32, dev)
    v_idx = torch.empty(max(vp[-1], 1), dtype=torch.int32, device=dev)
    s_idx = torch.empty(max(sp[-1], 1), dtype=torch.int32, device=dev)
    pv = _small_to_dev([float(x) for x in p_v], torch.float32, dev)
    ps = _small_to_dev([float(x) for x in p_s], torch.float32, dev)
    counts = torch.empty((len(vp) - 1, 2), dtype=torch.int32, device=dev)
    v_score = torch.empty((B, Hq, N), dtype=torch.float32, device=dev) if return_scores else None
    s_score = torch.empty((B, Hq, N // BLOCK), dtype=torch.float32, device=dev) if return_scores else None
    L = _abi.lib()
    nb = ctypes.c_size_t()
    _abi.check(L.vs_workspace_size(P.ref, 0, None, ctypes.byref(nb)))
    ws = _workspace(dev, nb.value)
    _abi.check(L.vs_estimate_index_topp(P.ref, _ptr(q), _ptr(k), 0, _ptr(pv), _ptr(ps), _ptr(v_ptr),
                                        _ptr(v_idx), _ptr(s_ptr), _ptr(s_idx), _ptr(counts),
                                        _ptr(v_score), _ptr(s_score), _ptr(ws), ws.numel(),
                                        _stream(dev)))
    idx = VsIndexT(v_ptr, v_idx, s_ptr, s_idx, vm, sm)
    return (idx, counts, v_score, s_score) if return_scores else (idx, counts)


def estimate_index_xattn(q: torch.Tensor, k: torch.Tensor, threshold: float = 0.9,
                         block: int = 128, stride: int = 16, return_scores: bool = False):
    """XAttention block selection for q [B, N, Hq, d], k [B, N, Hkv, d] bf16
    (one segment): 16-token cells scored along their anti-diagonals, a softmax
    over each cell row, block scores summed over cells, and per query block the
    fewest key blocks holding the share ``threshold`` of the row's score.

    Returns (VsIndexT with the block selection, counts [B, Hq, nI] int32) and,
    with return_scores, also the block scores [B, Hq, nI, nI] fp32 (entries of
    key blocks after the query block unspecified).
    """
    dev = q.device
    _need(q, "q", torch.bfloat16, dev, strided=True)
    _need(k, "k", torch.bfloat16, dev, strided=True)
    B, N, Hq, d = q.shape
    Hkv = k.shape[2]
    P = _Problem(B, Hq, Hkv, d, N, N, _abi.VS_BF16, None, None, None, q=q, k=k)
    nI = -(-N // block)
    mask = torch.empty((B * Hq * nI, -(-nI // 32)), dtype=torch.int32, device=dev)
    counts = torch.empty((B, Hq, nI), dtype=torch.int32, device=dev)
    scores = torch.empty((B, Hq, nI, nI), dtype=torch.float32, device=dev) if return_scores else None
    L = _abi.lib()
    nb = ctypes.c_size_t()
    _abi.check(L.vs_workspace_size(P.ref, 3, None, ctypes.byref(nb)))
    ws = _workspace(dev, nb.value)
    _abi.check(L.vs_estimate_index_xattn(P.ref, _ptr(q), _ptr(k), int(block), int(stride),
                                         float(threshold), _ptr(mask), _ptr(counts), _ptr(scores),
                                         _ptr(ws), ws.numel(), _stream(dev)))
    zeros = torch.zeros(B * Hq + 1, dtype=torch.int32, device=dev)
    empty = torch.zeros(1, dtype=torch.int32, device=dev)
    idx = VsIndexT(zeros, empty, zeros, empty, 0, 0, mask, int(block))
    return (idx, counts, scores) if return_scores else (idx, counts)


def estimate_index_moba(q: torch.Tensor, k: torch.Tensor, block: int = 4096, topk: int = 12,
                        return_scores: bool = False):
    """MoBA block gate for q [B, N, Hq, d], k [B, N, Hkv, d] bf16 (one
    segment): every query picks its own key block of `block` tokens and the
    topk - 1 earlier blocks whose mean key scores highest against it.

    Returns a VsIndexT with the per-row selection (row_mask [B, Hq, N] int32)
    and, with return_scores, also the gate scores [B, Hq, N, nB] fp32
    (entries of the own block and later unspecified).
    """
    dev = q.device
    _need(q, "q", torch.bfloat16, dev, strided=True)
    _need(k, "k", torch.bfloat16, dev, strided=True)
    B, N, Hq, d = q.shape
    Hkv = k.shape[2]
    P = _Problem(B, Hq, Hkv, d, N, N, _abi.VS_BF16, None, None, None, q=q, k=k)
    nB = -(-N // block)
    mask = torch.empty((B, Hq, N), dtype=torch.int32, device=dev)
    scores = torch.empty((B, Hq, N, nB), dtype=torch.float32, device=dev) if return_scores else None
    L = _abi.lib()
    nb = ctypes.c_size_t()
    _abi.check(L.vs_workspace_size(P.ref, 4, None, ctypes.byref(nb)))
    ws = _workspace(dev, nb.value)
    _abi.check(L.vs_estimate_index_moba(P.ref, _ptr(q), _ptr(k), int(block), int(topk), _ptr(mask),
                                        _ptr(scores), _ptr(ws), ws.numel(), _stream(dev)))
    zeros = torch.zeros(B * Hq + 1, dtype=torch.int32, device=dev)
    empty = torch.zeros(1, dtype=torch.int32, device=dev)
    idx = VsIndexT(zeros, empty, zeros, empty, 0, 0, row_mask=mask, row_blk=int(block))
    return (idx, scores) if return_scores else idx


def index_from_lists(lists: List[Tuple[Sequence[int], Sequence[int]]], device) -> VsIndexT:
    """Device index from host lists (list number l = (b*Hq + h)*n_seg + s)."""
    vp, sp, vi, si = [0], [0], [], []
    for v, s in lists:
        vi.extend(int(x) for x in v)
        si.extend(int(x) for x in s)
        vp.append(len(vi))
        sp.append(len(si))
    vm = max((vp[i + 1] - vp[i] for i in range(len(lists))), default=0)
    sm = max((sp[i + 1] - sp[i] for i in range(len(lists))), default=0)
    t = lambda x: torch.tensor(x if x else [0], dtype=torch.int32, device=device)
    return VsIndexT(t(vp), t(vi), t(sp), t(si), vm, sm)


def sparse_attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, index: VsIndexT,
                    cu_seqlens=None, stripe=None, o_f32: bool = False, scale=None,
                    out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                    merge: bool = False):
    """Sparse attention forward.  Returns (o [B, Nq, Hq, d], lse [B, Hq, Nq] fp32).

    stripe = (world, q_rank, k_rank) for a block-striped call (one ring step);
    k_rank = "all": k / v hold every rank's chunk, one after the other
    (the whole ring of worker q_rank in one call).
    merge: out (fp32) and lse hold a running result (zeros / -inf to start);
    this call's result is merged into them in place (fused lse_merge).
    """
    if merge:
        if out is None or lse is None:
            raise ValueError("merge needs out (fp32) and lse holding the running result")
        o_f32 = True
    dev = q.device
    _need(q, "q", dev=dev, strided=True)
    _need(k, "k", q.dtype, dev, strided=True)
    _need(v, "v", q.dtype, dev, strided=True)
    B, Nq, Hq, d = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    odt = torch.float32 if o_f32 else q.dtype
    o = out if out is not None else torch.empty((B, Nq, Hq, d), dtype=odt, device=dev)
    l = lse if lse is not None else torch.empty((B, Hq, Nq), dtype=torch.float32, device=dev)
    _need(o, "out", odt, dev, strided=True)
    _need(l, "lse", torch.float32, dev)
    P = _Problem(B, Hq, Hkv, d, Nq, Nk, _dtype_code(q), cu_seqlens, stripe, scale, q=q, k=k, v=v, o=o)
    ix = index.struct()
    L = _abi.lib()
    nb = ctypes.c_size_t()
    _abi.check(L.vs_workspace_size(P.ref, 1, ctypes.byref(ix), ctypes.byref(nb)))
    ws = _workspace(dev, nb.value)
    _abi.check(L.vs_sparse_attn_fwd(P.ref, _ptr(q), _ptr(k), _ptr(v), ctypes.byref(ix), _ptr(o),
                                    2 if merge else int(o_f32), _ptr(l), _ptr(ws), ws.numel(),
                                    _stream(dev)))
    return o, l


def attn_bwd_delta(o: torch.Tensor, do: torch.Tensor, out: Optional[torch.Tensor] = None):
    """delta [B, Hq, N] = rowsum(dO * O) (fp32)."""
    dev = do.device
    _need(o, "o", dev=dev, strided=True)
    _need(do, "do", dev=dev, strided=True)
    B, N, Hq, d = do.shape
    P = _Problem(B, Hq, Hq, d, N, N, _dtype_code(do), None, None, None, o=o, do=do)
    delta = out if out is not None else torch.empty((B, Hq, N), dtype=torch.float32, device=dev)
    _abi.check(_abi.lib().vs_attn_bwd_delta(P.ref, _ptr(o), int(o.dtype == torch.float32),
                                            _ptr(do), _ptr(delta), _stream(dev)))
    return delta


def sparse_attn_bwd_noalloc(q, k, v, o, do, lse, index: VsIndexT, delta=None, dq=None,
                            cu_seqlens=None, stripe=None, scale=None, dk=None, dv=None,
                            accumulate: bool = False):
    """sparse_attn_bwd through vs_sparse_attn_bwd_noalloc: the library's own
    per-GPU scratch array serves as the workspace (nothing is allocated for
    it; calls that overlap on one GPU race on it)."""
    return sparse_attn_bwd(q, k, v, o, do, lse, index, delta, dq, cu_seqlens, stripe, scale, dk, dv,
                           accumulate, _noalloc=True)


def sparse_attn_bwd(q, k, v, o, do, lse, index: VsIndexT, delta=None, dq=None,
                    cu_seqlens=None, stripe=None, scale=None, dk=None, dv=None,
                    accumulate: bool = False, _noalloc: bool = False):
    """Sparse attention backward.  Returns (dq, dk, dv), fp32.

    lse (and delta, if given) are the rows' final values.  dq / dk / dv are
    optional output buffers; with accumulate=True the gradient of Q is added
    to dq (chunked KV) instead of overwriting it.
    """
    dev = q.device
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (do, "do")):
        _need(t, n, q.dtype, dev, strided=True)
    _need(lse, "lse", torch.float32, dev)
    B, Nq, Hq, d = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    P = _Problem(B, Hq, Hkv, d, Nq, Nk, _dtype_code(q), cu_seqlens, stripe, scale, q=q, k=k, v=v, o=o, do=do)
    acc = bool(accumulate)
    if acc and dq is None:
        raise ValueError("accumulate=True needs dq")
    if dq is None:
        dq = torch.empty((B, Nq, Hq, d), dtype=torch.float32, device=dev)
    dk = dk if dk is not None else torch.empty((B, Nk, Hkv, d), dtype=torch.float32, device=dev)
    dv = dv if dv is not None else torch.empty((B, Nk, Hkv, d), dtype=torch.float32, device=dev)
    for t, n in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        _need(t, n, torch.float32, dev)
    o_f32 = 0
    if o is not None:
        _need(o, "o", dev=dev, strided=True)
        o_f32 = int(o.dtype == torch.float32)
    if delta is not None:
        _need(delta, "delta", torch.float32, dev)
    ix = index.struct()
    L = _abi.lib()
    if _noalloc:
        _abi.check(L.vs_sparse_attn_bwd_noalloc(P.ref, _ptr(q), _ptr(k), _ptr(v), _ptr(o), o_f32, _ptr(do),
                                                _ptr(lse), _ptr(delta), ctypes.byref(ix), _ptr(dq), int(acc),
                                                _ptr(dk), _ptr(dv), _stream(dev)))
        return dq, dk, dv
    nb = ctypes.c_size_t()
    _abi.check(L.vs_workspace_size(P.ref, 2, ctypes.byref(ix), ctypes.byref(nb)))
    ws = _workspace(dev, nb.value)
    _abi.check(L.vs_sparse_attn_bwd(P.ref, _ptr(q), _ptr(k), _ptr(v), _ptr(o), o_f32, _ptr(do),
                                    _ptr(lse), _ptr(delta), ctypes.byref(ix), _ptr(dq), int(acc),
                                    _ptr(dk), _ptr(dv), _ptr(ws), ws.numel(), _stream(dev)))
    return dq, dk, dv


def lse_merge(o_acc: torch.Tensor, lse_acc: torch.Tensor, o_part: torch.Tensor,
              lse_part: torch.Tensor):
    """In-place merge of a partial (o_part, lse_part) into (o_acc, lse_acc); fp32, BSHD / BHS."""
    dev = o_acc.device
    for t, n in ((o_acc, "o_acc"), (lse_acc, "lse_acc"), (o_part, "o_part"), (lse_part, "lse_part")):
        _need(t, n, torch.float32, dev)
    B, N, H, d = o_acc.shape
    if o_part.shape != o_acc.shape or lse_acc.shape != (B, H, N) or lse_part.shape != (B, H, N):
        raise ValueError("lse_merge shapes disagree")
    _abi.check(_abi.lib().lse_merge(B, N, H, d, _ptr(o_acc), _ptr(lse_acc), _ptr(o_part),
                                    _ptr(lse_part), _stream(dev)))
    return o_acc, lse_acc
