"""ctypes binding of ``libjssa.so`` (the C ABI in ``include/jssa.h``).

Argument marshalling only: descriptors become ``jssa_desc`` structs, torch
tensors become their device pointers, the current HIP stream is passed
through, and a non-zero status raises :class:`JssaError`.  Every step of the
decode path runs in the library's HIP kernels; nothing here computes.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libjssa.so")

F32, BF16, FP8_E4M3 = 0, 1, 2  # FP8_E4M3: projected-key caches only (uint8 codes)
REDUCE_MAX, REDUCE_MEAN = 0, 1
LAYOUT_GQA, LAYOUT_MLA = 0, 1
OP_TOPK, OP_ATTN, OP_DECODE, OP_DENSE, OP_SCORE, OP_VOTE = 1, 2, 3, 4, 5, 6

STATUS = {0: "JSSA_OK", -1: "JSSA_ERR_INVALID_ARG", -2: "JSSA_ERR_UNSUPPORTED",
          -3: "JSSA_ERR_WORKSPACE", -4: "JSSA_ERR_MISALIGNED", -5: "JSSA_ERR_HIP", -6: "JSSA_ERR_TOO_LARGE"}

# every function include/jssa.h declares, with its ctypes signature
_c_void_p, _i32, _size_t = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t


class CDesc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "n_q_heads", "n_kv_heads", "d_k", "d_v", "rank", "t_max", "topk", "window",
        "kv_dtype", "kp_dtype", "out_dtype", "reduce", "layout")] + [("scale", ctypes.c_float)]


_PDESC = ctypes.POINTER(CDesc)
SIGNATURES = {
    "jssa_abi_version": (_i32, []),
    "jssa_status_str": (ctypes.c_char_p, [_i32]),
    "jssa_check_desc": (_i32, [_PDESC, _i32]),
    "jssa_workspace_bytes": (_size_t, [_PDESC, _i32]),
    "jssa_workspace_init": (_i32, [_c_void_p, _size_t, _c_void_p]),
    "jssa_workspace_status": (_i32, [_c_void_p, _size_t, _c_void_p, _i32, _c_void_p]),
    "jssa_append_kv": (_i32, [_PDESC, _c_void_p, _c_void_p, _i32, _c_void_p, _c_void_p,
                              _c_void_p, _c_void_p, _c_void_p, _c_void_p]),
    "jssa_score": (_i32, [_PDESC, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                          _size_t, _c_void_p]),
    "jssa_topk": (_i32, [_PDESC, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _size_t,
                         _c_void_p]),
    "jssa_indexed_attn": (_i32, [_PDESC, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                 _c_void_p, _c_void_p, _c_void_p, _size_t, _c_void_p]),
    "jssa_decode": (_i32, [_PDESC, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                           _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                           _size_t, _c_void_p]),
    "jssa_decode_profiled": (_i32, [_PDESC, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                    _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                    _size_t, ctypes.POINTER(_c_void_p), _c_void_p]),
    "jssa_decode_step": (_i32, [_PDESC, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                _c_void_p, _c_void_p, _c_void_p, _size_t, ctypes.POINTER(_c_void_p),
                                _c_void_p]),
    "jssa_decode_step_static": (_i32, [_PDESC, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                       _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                       _c_void_p, _c_void_p, _c_void_p]),
    "jssa_reuse_step": (_i32, [_PDESC, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                               _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _size_t, _c_void_p]),
    "jssa_vote_select": (_i32, [_PDESC, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _size_t,
                                _c_void_p]),
    "jssa_gather_kv": (_i32, [_PDESC, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                              _c_void_p, _c_void_p]),
    "jssa_dense_decode": (_i32, [_PDESC, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                 _c_void_p, _c_void_p, _size_t, _c_void_p]),
}


class JssaError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} returned {STATUS.get(status, status)}")
        self.status = status


_lib = None


def lib():
    """The loaded library; raises if it has not been built (no fallback path exists)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise ImportError(f"{_LIB_PATH} is missing: build it with "
                              "`python -m token_level_sparse_dim_amd.build`")
        h = ctypes.CDLL(_LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(h, name)
            fn.restype = res
            fn.argtypes = args
        _lib = h
    return _lib


@dataclass(frozen=True)
class Desc:
    """Python mirror of ``jssa_desc``."""
    batch: int
    n_q_heads: int
    n_kv_heads: int
    d_k: int
    d_v: int
    rank: int
    t_max: int
    topk: int
    window: int = 0
    kv_dtype: int = BF16
    kp_dtype: int = BF16
    out_dtype: int = F32
    reduce: int = REDUCE_MAX
    layout: int = LAYOUT_GQA
    scale: float = 0.0

    def c(self) -> CDesc:
        return CDesc(self.batch, self.n_q_heads, self.n_kv_heads, self.d_k, self.d_v, self.rank,
                     self.t_max, self.topk, self.window, self.kv_dtype, self.kp_dtype,
                     self.out_dtype, self.reduce, self.layout, float(self.scale))


def call(name: str, *args) -> None:
    st = getattr(lib(), name)(*args)
    if st != 0:
        raise JssaError(name, st)
