"""ctypes view of the C ABI in include/vs.h (argument marshalling only)."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libvs.so")

VS_OK = 0
VS_ERR_NULL = -1
VS_ERR_SHAPE = -2
VS_ERR_UNSUPPORTED = -3
VS_ERR_BUDGET = -4
VS_ERR_WORKSPACE = -5
VS_ERR_HIP = -6
VS_ERR_INDEX = -7
VS_F32 = 0
VS_BF16 = 1
VS_MAX_SEGMENTS = 128

# Every function the header declares, with its ctypes signature.
i32, f32, vp, sz = ctypes.c_int32, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t
i32p = ctypes.POINTER(ctypes.c_int32)


VS_ALL_CHUNKS = -1
i64x3 = ctypes.c_int64 * 3


class VsProblem(ctypes.Structure):
    _fields_ = [("batch", i32), ("h_q", i32), ("h_kv", i32), ("head_dim", i32), ("n_q", i32),
                ("n_k", i32), ("block", i32), ("dtype", i32), ("scale", f32), ("n_seg", i32),
                ("cu_seqlens", i32p), ("stripe_world", i32), ("q_rank", i32), ("k_rank", i32),
                ("q_stride", i64x3), ("k_stride", i64x3), ("v_stride", i64x3), ("o_stride", i64x3),
                ("do_stride", i64x3)]


class VsIndex(ctypes.Structure):
    _fields_ = [("v_ptr", vp), ("v_idx", vp), ("s_ptr", vp), ("s_idx", vp), ("v_cap_max", i32),
                ("s_cap_max", i32), ("blk_mask", vp), ("blk_size", i32), ("row_mask", vp), ("row_blk", i32)]


PP = ctypes.POINTER(VsProblem)
IP = ctypes.POINTER(VsIndex)

SIGNATURES = {
    "vs_index_capacity": (i32, [PP, i32p, i32p, i32p, i32p, i32p, i32p]),
    "vs_workspace_size": (i32, [PP, i32, IP, ctypes.POINTER(sz)]),
    "vs_estimate_index": (i32, [PP, vp, vp, i32, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
    "vs_estimate_index_topp": (i32, [PP, vp, vp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
    "vs_estimate_index_xattn": (i32, [PP, vp, vp, i32, i32, f32, vp, vp, vp, vp, sz, vp]),
    "vs_estimate_index_moba": (i32, [PP, vp, vp, i32, i32, vp, vp, vp, sz, vp]),
    "vs_sparse_attn_fwd": (i32, [PP, vp, vp, vp, IP, vp, i32, vp, vp, sz, vp]),
    "vs_attn_bwd_delta": (i32, [PP, vp, i32, vp, vp, vp]),
    "vs_sparse_attn_bwd": (i32, [PP, vp, vp, vp, vp, i32, vp, vp, vp, IP, vp, i32, vp, vp, vp, sz, vp]),
    "vs_sparse_attn_bwd_noalloc": (i32, [PP, vp, vp, vp, vp, i32, vp, vp, vp, IP, vp, i32, vp, vp, vp]),
    "lse_merge": (i32, [i32, i32, i32, i32, vp, vp, vp, vp, vp]),
    "vs_trace_enable": (i32, [i32]),
    "vs_trace_collect": (i32, [ctypes.c_char_p, sz]),
    "vs_last_error": (ctypes.c_char_p, []),
}

_lib = None


class VsError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"vs status {status}: {message}")
        self.status = status


def lib():
    """The loaded libvs.so; raises if it has not been built (no fallback exists)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m dynamic_sparse_attention_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def check(status: int):
    if status != VS_OK:
        raise VsError(status, lib().vs_last_error().decode(errors="replace"))
