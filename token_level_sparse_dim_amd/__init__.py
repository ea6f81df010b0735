"""MI355X (gfx950) token-level sparse decode attention: Python binding.

Thin wrappers with the C ABI's names (``include/jssa.h``).  Tensors are
device tensors owned by the caller; the functions pass their pointers and the
current HIP stream to ``libjssa.so`` and raise :class:`JssaError` on a
non-zero status.  PyTorch provides device memory and streams only.
"""
from __future__ import annotations

import torch

from ._lib import (BF16, F32, FP8_E4M3, LAYOUT_GQA, LAYOUT_MLA, OP_ATTN, OP_DECODE, OP_DENSE, OP_SCORE,
                   OP_TOPK, OP_VOTE,
                   REDUCE_MAX, REDUCE_MEAN, Desc, JssaError, call, lib)

__all__ = [
    "Desc", "JssaError", "F32", "BF16", "FP8_E4M3", "REDUCE_MAX", "REDUCE_MEAN", "LAYOUT_GQA", "LAYOUT_MLA",
    "OP_TOPK", "OP_ATTN", "OP_DECODE", "OP_DENSE", "OP_SCORE", "OP_VOTE", "lib", "abi_version", "check_desc",
    "workspace_bytes", "workspace", "workspace_status", "STATUS_WAIT_TIMEOUT", "STATUS_EXACT_REDO",
    "STATUS_RANGE_SPLIT", "STATUS_GLOBAL_CUT", "append_kv", "append_projection", "score", "topk", "indexed_attn", "decode", "decode_profiled",
    "decode_step", "decode_step_static", "reuse_step", "vote_select", "gather_kv", "dense_decode",
]

# FP8 E4M3 projected keys travel as their byte codes
_TORCH_DTYPE = {F32: torch.float32, BF16: torch.bfloat16, FP8_E4M3: torch.uint8}


def _ptr(t, dtype=None, name="tensor"):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    return t.data_ptr()


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def abi_version() -> int:
    return int(lib().jssa_abi_version())


def check_desc(desc: Desc, op: int = 0) -> int:
    """Status the library reports for ``desc`` and ``op`` (0 = append/score)."""
    d = desc.c()
    return int(lib().jssa_check_desc(d, op))


def workspace_bytes(desc: Desc, op: int) -> int:
    d = desc.c()
    return int(lib().jssa_workspace_bytes(d, op))


def workspace(desc: Desc, op: int, device="cuda", stream=None) -> torch.Tensor:
    """A zero-initialised workspace for ``op`` (a uint8 device tensor)."""
    n = workspace_bytes(desc, op)
    if n == 0:
        raise JssaError("jssa_workspace_bytes", -1)
    ws = torch.empty(n, dtype=torch.uint8, device=device)
    call("jssa_workspace_init", _ptr(ws, torch.uint8, "ws"), n, _stream(stream))
    return ws


STATUS_WAIT_TIMEOUT, STATUS_EXACT_REDO, STATUS_RANGE_SPLIT, STATUS_GLOBAL_CUT = 0, 1, 2, 3


def workspace_status(ws, clear: bool = True, out=None, stream=None) -> torch.Tensor:
    """``jssa_workspace_status``: the workspace's diagnostic words, copied into a
    4-element int32 device tensor (``out`` or a new one) on the stream and, with
    ``clear``, reset.  Index with ``STATUS_WAIT_TIMEOUT`` (nonzero: a bounded
    in-kernel wait gave up, results since the last clear are wrong),
    ``STATUS_EXACT_REDO``, ``STATUS_RANGE_SPLIT`` and ``STATUS_GLOBAL_CUT`` (counts)."""
    if out is None:
        out = torch.zeros(4, dtype=torch.int32, device=ws.device)
    call("jssa_workspace_status", _ptr(ws, torch.uint8, "ws"), ws.numel(), _ptr(out, torch.int32, "out"),
         1 if clear else 0, _stream(stream))
    return out


def append_kv(desc: Desc, k_new, v_new, pos, P, k_cache, v_cache, kp_cache, stream=None):
    """``jssa_append_kv``: write new K/V rows ``[B, n_new, Hkv, d]`` at ``pos`` and
    project their keys into the scoring cache."""
    kv, kp = _TORCH_DTYPE[desc.kv_dtype], _TORCH_DTYPE[desc.kp_dtype]
    n_new = k_new.shape[1]
    call("jssa_append_kv", desc.c(), _ptr(k_new, kv, "k_new"), _ptr(v_new, kv, "v_new"), int(n_new),
         _ptr(pos, torch.int32, "pos"), _ptr(P, torch.float32, "P"), _ptr(k_cache, kv, "k_cache"),
         _ptr(v_cache, kv, "v_cache"), _ptr(kp_cache, kp, "kp_cache"), _stream(stream))


def append_projection(desc: Desc, n_new: int, pos, P, k_cache, kp_cache, stream=None):
    """``jssa_append_kv`` with ``k_new = NULL``: project ``n_new`` cached rows from ``pos``."""
    kv, kp = _TORCH_DTYPE[desc.kv_dtype], _TORCH_DTYPE[desc.kp_dtype]
    call("jssa_append_kv", desc.c(), None, None, int(n_new), _ptr(pos, torch.int32, "pos"),
         _ptr(P, torch.float32, "P"), _ptr(k_cache, kv, "k_cache"), None,
         _ptr(kp_cache, kp, "kp_cache"), _stream(stream))


def score(desc: Desc, q, P, kp_cache, seq_lens, scores, ws=None, stream=None):
    """``jssa_score``: subspace scores of every candidate token.  ``ws`` is the
    JSSA_OP_SCORE workspace; MLA descriptors need one (GQA ones ignore it)."""
    wsp, wsn = (None, 0) if ws is None else (_ptr(ws, torch.uint8, "ws"), ws.numel())
    call("jssa_score", desc.c(), _ptr(q, _TORCH_DTYPE[desc.kv_dtype], "q"), _ptr(P, torch.float32, "P"),
         _ptr(kp_cache, _TORCH_DTYPE[desc.kp_dtype], "kp_cache"), _ptr(seq_lens, torch.int32, "seq_lens"),
         _ptr(scores, torch.float32, "scores"), wsp, wsn, _stream(stream))


def topk(desc: Desc, scores, seq_lens, idx, n_sel, ws, stream=None):
    """``jssa_topk``: exact per-(sequence, KV head) selection plus the window."""
    call("jssa_topk", desc.c(), _ptr(scores, torch.float32, "scores"), _ptr(seq_lens, torch.int32, "seq_lens"),
         _ptr(idx, torch.int32, "idx"), _ptr(n_sel, torch.int32, "n_sel"), _ptr(ws, torch.uint8, "ws"),
         ws.numel(), _stream(stream))


def indexed_attn(desc: Desc, q, k_cache, v_cache, idx, n_sel, out, lse, ws, stream=None):
    """``jssa_indexed_attn``: gather-free attention over the selected rows."""
    kv = _TORCH_DTYPE[desc.kv_dtype]
    call("jssa_indexed_attn", desc.c(), _ptr(q, kv, "q"), _ptr(k_cache, kv, "k_cache"),
         _ptr(v_cache, kv, "v_cache"), _ptr(idx, torch.int32, "idx"), _ptr(n_sel, torch.int32, "n_sel"),
         _ptr(out, _TORCH_DTYPE[desc.out_dtype], "out"), _ptr(lse, torch.float32, "lse"),
         _ptr(ws, torch.uint8, "ws"), ws.numel(), _stream(stream))


def decode(desc: Desc, q, P, kp_cache, k_cache, v_cache, seq_lens, out, lse, ws,
           idx_out=None, n_sel_out=None, stream=None):
    """``jssa_decode``: score -> top-k -> indexed attention in one call."""
    kv = _TORCH_DTYPE[desc.kv_dtype]
    call("jssa_decode", desc.c(), _ptr(q, kv, "q"), _ptr(P, torch.float32, "P"),
         _ptr(kp_cache, _TORCH_DTYPE[desc.kp_dtype], "kp_cache"), _ptr(k_cache, kv, "k_cache"),
         _ptr(v_cache, kv, "v_cache"), _ptr(seq_lens, torch.int32, "seq_lens"),
         _ptr(out, _TORCH_DTYPE[desc.out_dtype], "out"), _ptr(lse, torch.float32, "lse"),
         _ptr(idx_out, torch.int32, "idx_out"), _ptr(n_sel_out, torch.int32, "n_sel_out"),
         _ptr(ws, torch.uint8, "ws"), ws.numel(), _stream(stream))


def decode_profiled(desc: Desc, q, P, kp_cache, k_cache, v_cache, seq_lens, out, lse, ws, events,
                    idx_out=None, n_sel_out=None, stream=None):
    """``jssa_decode_profiled``: :func:`decode` recording four stage events
    (``torch.cuda.Event(enable_timing=True)``) around its launches; the fused
    build records them as the scan launch's own start and end, then after the
    select/attend launch and right after that (the header lists the staged
    shapes' points)."""
    arr = _event_array(events, stream)
    kv = _TORCH_DTYPE[desc.kv_dtype]
    call("jssa_decode_profiled", desc.c(), _ptr(q, kv, "q"), _ptr(P, torch.float32, "P"),
         _ptr(kp_cache, _TORCH_DTYPE[desc.kp_dtype], "kp_cache"), _ptr(k_cache, kv, "k_cache"),
         _ptr(v_cache, kv, "v_cache"), _ptr(seq_lens, torch.int32, "seq_lens"),
         _ptr(out, _TORCH_DTYPE[desc.out_dtype], "out"), _ptr(lse, torch.float32, "lse"),
         _ptr(idx_out, torch.int32, "idx_out"), _ptr(n_sel_out, torch.int32, "n_sel_out"),
         _ptr(ws, torch.uint8, "ws"), ws.numel(), arr, _stream(stream))


def _event_array(events, stream):
    """A host array of the four events' HIP handles (torch creates an event on
    its first record, so unrecorded events are recorded once here first)."""
    import ctypes
    if len(events) != 4:
        raise ValueError("four events are needed")
    for e in events:
        if not e.cuda_event:
            e.record(stream if stream is not None else torch.cuda.current_stream())
    return (ctypes.c_void_p * 4)(*[ctypes.c_void_p(e.cuda_event) for e in events])


def decode_step(desc: Desc, k_new, v_new, pos, q, P, kp_cache, k_cache, v_cache, seq_lens, out, lse, ws,
                idx_out=None, n_sel_out=None, events=None, stream=None):
    """``jssa_decode_step``: append one new token per sequence (``k_new`` /
    ``v_new`` ``[B, 1, Hkv, d]`` at ``pos``), then the decode on the updated
    caches; the result of :func:`append_kv` followed by :func:`decode`.
    ``events``: optional four stage events, as for :func:`decode_profiled`."""
    kv = _TORCH_DTYPE[desc.kv_dtype]
    if k_new.shape[1] != 1:
        raise ValueError("decode_step appends exactly one token per sequence")
    arr = None if events is None else _event_array(events, stream)
    call("jssa_decode_step", desc.c(), _ptr(k_new, kv, "k_new"), _ptr(v_new, kv, "v_new"),
         _ptr(pos, torch.int32, "pos"), _ptr(q, kv, "q"), _ptr(P, torch.float32, "P"),
         _ptr(kp_cache, _TORCH_DTYPE[desc.kp_dtype], "kp_cache"), _ptr(k_cache, kv, "k_cache"),
         _ptr(v_cache, kv, "v_cache"), _ptr(seq_lens, torch.int32, "seq_lens"),
         _ptr(out, _TORCH_DTYPE[desc.out_dtype], "out"), _ptr(lse, torch.float32, "lse"),
         _ptr(idx_out, torch.int32, "idx_out"), _ptr(n_sel_out, torch.int32, "n_sel_out"),
         _ptr(ws, torch.uint8, "ws"), ws.numel(), arr, _stream(stream))


def decode_step_static(desc: Desc, k_new, v_new, pos, q, P, kp_cache, k_cache, v_cache, seq_lens, out, lse,
                       idx_out=None, n_sel_out=None, stream=None):
    """``jssa_decode_step_static``: :func:`decode_step` without a workspace (the
    library's static device scratch holds the intermediates; nothing is
    allocated).  Calls that overlap on one GPU race."""
    kv = _TORCH_DTYPE[desc.kv_dtype]
    if k_new.shape[1] != 1:
        raise ValueError("decode_step_static appends exactly one token per sequence")
    call("jssa_decode_step_static", desc.c(), _ptr(k_new, kv, "k_new"), _ptr(v_new, kv, "v_new"),
         _ptr(pos, torch.int32, "pos"), _ptr(q, kv, "q"), _ptr(P, torch.float32, "P"),
         _ptr(kp_cache, _TORCH_DTYPE[desc.kp_dtype], "kp_cache"), _ptr(k_cache, kv, "k_cache"),
         _ptr(v_cache, kv, "v_cache"), _ptr(seq_lens, torch.int32, "seq_lens"),
         _ptr(out, _TORCH_DTYPE[desc.out_dtype], "out"), _ptr(lse, torch.float32, "lse"),
         _ptr(idx_out, torch.int32, "idx_out"), _ptr(n_sel_out, torch.int32, "n_sel_out"), _stream(stream))


def reuse_step(desc: Desc, k_new, v_new, pos, q, k_cache, v_cache, idx, n_sel, out, lse, ws, stream=None):
    """``jssa_reuse_step``: one decode step of a layer that reuses an indexer
    layer's selection: the new token's K/V rows (``[B, 1, Hkv, d]`` at
    ``pos``; ``k_new=None``: none) are written without projection, then the
    indexed attention over ``idx`` / ``n_sel``. Workspace op ``OP_DECODE``."""
    kv = _TORCH_DTYPE[desc.kv_dtype]
    if k_new is not None and k_new.shape[1] != 1:
        raise ValueError("reuse_step appends exactly one token per sequence")
    call("jssa_reuse_step", desc.c(), _ptr(k_new, kv, "k_new"), _ptr(v_new, kv, "v_new"),
         _ptr(pos, torch.int32, "pos"), _ptr(q, kv, "q"), _ptr(k_cache, kv, "k_cache"),
         _ptr(v_cache, kv, "v_cache"), _ptr(idx, torch.int32, "idx"), _ptr(n_sel, torch.int32, "n_sel"),
         _ptr(out, _TORCH_DTYPE[desc.out_dtype], "out"), _ptr(lse, torch.float32, "lse"),
         _ptr(ws, torch.uint8, "ws"), ws.numel(), _stream(stream))


def vote_select(desc: Desc, scores, seq_lens, idx, n_sel, ws, stream=None):
    """``jssa_vote_select``: head-shared soft-voting selection: one top-k of
    the KV heads' summed softmax votes per sequence, written to every KV
    head's list (``idx`` ``[B, Hkv, k + W]``, ``n_sel`` ``[B, Hkv]``)."""
    call("jssa_vote_select", desc.c(), _ptr(scores, torch.float32, "scores"),
         _ptr(seq_lens, torch.int32, "seq_lens"), _ptr(idx, torch.int32, "idx"),
         _ptr(n_sel, torch.int32, "n_sel"), _ptr(ws, torch.uint8, "ws"), ws.numel(), _stream(stream))


def gather_kv(desc: Desc, k_cache, v_cache, idx, n_sel, k_packed, v_packed, packed_lens=None, stream=None):
    """``jssa_gather_kv``: pack the selected K/V rows into ``[B, topk + window,
    Hkv, d]`` buffers (the gather-then-attend baseline); ``packed_lens``
    receives the per-sequence counts for :func:`dense_decode` on them."""
    kv = _TORCH_DTYPE[desc.kv_dtype]
    call("jssa_gather_kv", desc.c(), _ptr(k_cache, kv, "k_cache"), _ptr(v_cache, kv, "v_cache"),
         _ptr(idx, torch.int32, "idx"), _ptr(n_sel, torch.int32, "n_sel"), _ptr(k_packed, kv, "k_packed"),
         _ptr(v_packed, kv, "v_packed"), _ptr(packed_lens, torch.int32, "packed_lens"), _stream(stream))


def dense_decode(desc: Desc, q, k_cache, v_cache, seq_lens, out, lse, ws, stream=None):
    """``jssa_dense_decode``: full-KV decode attention (comparison path)."""
    kv = _TORCH_DTYPE[desc.kv_dtype]
    call("jssa_dense_decode", desc.c(), _ptr(q, kv, "q"), _ptr(k_cache, kv, "k_cache"),
         _ptr(v_cache, kv, "v_cache"), _ptr(seq_lens, torch.int32, "seq_lens"),
         _ptr(out, _TORCH_DTYPE[desc.out_dtype], "out"), _ptr(lse, torch.float32, "lse"),
         _ptr(ws, torch.uint8, "ws"), ws.numel(), _stream(stream))
