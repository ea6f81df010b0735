"""The C-ABI library: it loads, exports every function include/jssa.h declares,
and rejects bad arguments on the host before touching the GPU (CPU only)."""
import ctypes
import os
import re

import pytest

import token_level_sparse_dim_amd as J
from token_level_sparse_dim_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "jssa.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(jssa_[a-z_]+)\s*\(", src)))


def _desc(**kw):
    base = dict(batch=2, n_q_heads=32, n_kv_heads=8, d_k=128, d_v=128, rank=32, t_max=8192,
                topk=256, window=0, kv_dtype=J.BF16, kp_dtype=J.BF16, out_dtype=J.F32,
                reduce=J.REDUCE_MAX, layout=J.LAYOUT_GQA, scale=128 ** -0.5)
    base.update(kw)
    return J.Desc(**base)


def test_library_exports_every_declared_function():
    names = _declared()
    assert len(names) >= 11
    lib = J.lib()
    for n in names:
        assert hasattr(lib, n), n
        assert n in _lib.SIGNATURES, n
    assert set(_lib.SIGNATURES) == set(names)


def test_abi_version_and_status_strings():
    assert J.abi_version() == 10
    lib = J.lib()
    assert lib.jssa_status_str(0) == b"JSSA_OK"
    for code, name in _lib.STATUS.items():
        assert lib.jssa_status_str(code).decode() == name
    assert lib.jssa_status_str(-99) == b"JSSA_ERR_UNKNOWN"


def test_struct_layout_matches_header():
    # 14 int32 fields and one float, no padding
    assert ctypes.sizeof(_lib.CDesc) == 15 * 4


@pytest.mark.parametrize("kw,status", [
    (dict(), 0),
    (dict(n_q_heads=30), -1),           # Hq not a multiple of Hkv
    (dict(batch=0), -1),
    (dict(t_max=0), -1),
    (dict(t_max=(1 << 24) + 1), -1),
    (dict(topk=-1), -1),
    (dict(kv_dtype=7), -1),
    (dict(reduce=5), -1),
    (dict(scale=float("nan")), -1),
    (dict(rank=48), -2),                # not built
    (dict(d_k=96, d_v=96), -2),
    (dict(d_v=64), -2),
    (dict(n_q_heads=48, n_kv_heads=3), -2),  # G = 16
    (dict(rank=256, d_k=128), -1),     # rank > d_k
    (dict(kp_dtype=J.FP8_E4M3), 0),     # FP8 projected keys, rank 32
    (dict(kp_dtype=J.FP8_E4M3, rank=64), 0),
    (dict(kp_dtype=J.FP8_E4M3, rank=16), -2),  # FP8 keys are scored on the matrix cores only
    (dict(kp_dtype=J.FP8_E4M3, kv_dtype=J.F32), -2),
    (dict(kv_dtype=J.FP8_E4M3), -1),    # q, K and V are never FP8
    (dict(out_dtype=J.FP8_E4M3), -1),
    (dict(kp_dtype=3), -1),
])
def test_descriptor_validation(kw, status):
    assert J.check_desc(_desc(**kw), J.OP_DECODE) == status


def test_selection_needs_a_budget_or_window():
    d = _desc(topk=0, window=0)
    assert J.check_desc(d, J.OP_TOPK) == -1
    assert J.check_desc(d, J.OP_DENSE) == 0
    assert J.check_desc(_desc(topk=0, window=16), J.OP_DECODE) == 0


def test_workspace_sizes():
    d = _desc()
    for op in (J.OP_TOPK, J.OP_ATTN, J.OP_DECODE, J.OP_DENSE, J.OP_SCORE, J.OP_VOTE):
        n = J.workspace_bytes(d, op)
        assert n > 0 and n % 256 == 0
    slots = d.batch * d.n_kv_heads * d.t_max * 8  # candidate slots: 8 bytes per token and row
    assert J.workspace_bytes(d, J.OP_DECODE) > slots and J.workspace_bytes(d, J.OP_TOPK) > slots
    # the fused decode keeps no per-token score array; the staged decode (G = 2 in bf16) does
    staged = _desc(n_q_heads=16)
    assert J.workspace_bytes(staged, J.OP_DECODE) > J.workspace_bytes(staged, J.OP_TOPK) + slots // 2
    assert J.workspace_bytes(_desc(n_q_heads=30), J.OP_DECODE) == 0
    assert J.workspace_bytes(d, 99) == 0


def _fake(n=1):
    return [ctypes.c_void_p(4096 * (i + 1)) for i in range(n)]


def test_entry_points_reject_bad_arguments_before_launch():
    lib = J.lib()
    d = _desc().c()
    p = _fake(12)
    null = None
    # null required pointers
    assert lib.jssa_score(d, null, *p[:4], null, 0, null) == -1
    assert lib.jssa_topk(d, *p[:4], null, 0, null) == -3            # workspace missing
    assert lib.jssa_topk(d, *p[:4], ctypes.c_void_p(4096), 16, null) == -3  # too small
    assert lib.jssa_topk(d, *p[:4], ctypes.c_void_p(4096 + 16), 1 << 40, null) == -3  # misaligned ws
    assert lib.jssa_indexed_attn(d, *p[:5], null, null, null, 0, null) == -1
    assert lib.jssa_decode(d, *p[:6], null, null, null, null, null, 0, null) == -1
    assert lib.jssa_dense_decode(d, null, *p[:4], null, null, 0, null) == -1
    assert lib.jssa_append_kv(d, *p[:2], -1, *p[2:7], null) == -1
    assert lib.jssa_vote_select(d, *p[:3], null, p[10], 1 << 40, null) == -1
    assert lib.jssa_vote_select(d, *p[:4], null, 0, null) == -3  # workspace missing
    assert lib.jssa_vote_select(_mla().c(), *p[:4], p[10], 1 << 40, null) == -2  # MLA: one set already
    assert lib.jssa_gather_kv(d, p[0], null, *p[2:6], null, null) == -1  # GQA needs V
    assert lib.jssa_gather_kv(d, *p[:3], null, *p[4:6], null, null) == -1
    assert lib.jssa_gather_kv(d, *p[:5], ctypes.c_void_p(4096 + 4), null, null) == -4
    # decode step: the new token's rows and positions are required (GQA: v_new and v_cache too)
    tail = (null, null, null, p[10], 1 << 40, null, null)  # lse, idx, n_sel, ws, ws_bytes, events, stream
    assert lib.jssa_decode_step(d, null, *p[:9], *tail) == -1
    assert lib.jssa_decode_step(d, p[0], p[1], null, *p[3:10], *tail) == -1
    assert lib.jssa_decode_step(d, p[0], null, *p[2:10], *tail) == -1
    assert lib.jssa_decode_step(d, *p[:10], null, null, null, null, 0, null, null) == -3  # workspace missing
    # reuse step: q, the caches, the lists and out are required; the new rows
    # need their positions (GQA: and v_new); k_new NULL appends nothing
    rs = (p[10], 1 << 40, null)  # ws, ws_bytes, stream
    assert lib.jssa_reuse_step(d, *p[:3], null, *p[4:9], null, *rs) == -1
    assert lib.jssa_reuse_step(d, p[0], p[1], null, *p[3:9], null, *rs) == -1
    assert lib.jssa_reuse_step(d, p[0], null, *p[2:9], null, *rs) == -1
    assert lib.jssa_reuse_step(d, *p[:7], null, p[8], null, *rs) == -1
    assert lib.jssa_reuse_step(d, *p[:9], null, null, 0, null) == -3  # workspace missing
    assert lib.jssa_reuse_step(d, null, null, null, *p[3:9], null, null, 0, null) == -3
    assert lib.jssa_reuse_step(d, *p[:8], ctypes.c_void_p(4096 + 2), null, *rs) == -4
    assert lib.jssa_reuse_step(_mla().c(), p[0], null, p[2], p[3], p[4], null, *p[6:9], null, null, 0,
                               null) == -3  # MLA: no V
    # misaligned data pointers
    odd = ctypes.c_void_p(4096 + 2)
    assert lib.jssa_score(d, odd, *p[:4], null, 0, null) == -4
    assert lib.jssa_decode(d, *p[:5], odd, p[6], null, null, null, p[7], 1 << 40, null) == -4
    assert lib.jssa_decode_step(d, odd, *p[1:10], *tail) == -4
    assert lib.jssa_decode_step(d, p[0], p[1], odd, *p[3:10], *tail) == -4
    # invalid descriptor wins over everything else
    bad = _desc(n_q_heads=30).c()
    assert lib.jssa_decode(bad, *p[:7], null, null, null, p[7], 1 << 40, null) == -1
    assert lib.jssa_score(None, *p[:5], null, 0, null) == -1
    # workspace init argument checks
    assert lib.jssa_workspace_init(None, 64, None) == -1
    assert lib.jssa_workspace_init(ctypes.c_void_p(4096 + 8), 64, None) == -3
    assert lib.jssa_workspace_init(None, 0, None) == 0  # nothing to do
    # workspace status: the workspace and the output are required; the
    # workspace holds at least its 256-byte queue region, 256-byte aligned
    assert lib.jssa_workspace_status(None, 256, p[0], 1, None) == -1
    assert lib.jssa_workspace_status(p[0], 256, None, 1, None) == -1
    assert lib.jssa_workspace_status(ctypes.c_void_p(4096 + 16), 256, p[1], 1, None) == -3
    assert lib.jssa_workspace_status(p[0], 128, p[1], 1, None) == -3
    assert lib.jssa_workspace_status(p[0], 256, ctypes.c_void_p(4096 + 4), 1, None) == -4


def test_status_words_match_header():
    src = open(HEADER).read()
    for name, val in (("JSSA_STATUS_WORDS", 4), ("JSSA_STATUS_WAIT_TIMEOUT", J.STATUS_WAIT_TIMEOUT),
                      ("JSSA_STATUS_EXACT_REDO", J.STATUS_EXACT_REDO),
                      ("JSSA_STATUS_RANGE_SPLIT", J.STATUS_RANGE_SPLIT),
                      ("JSSA_STATUS_GLOBAL_CUT", J.STATUS_GLOBAL_CUT)):
        assert re.search(rf"#define {name} {val}\b", src), name


def _mla(**kw):
    base = dict(batch=8, n_q_heads=128, n_kv_heads=1, d_k=576, d_v=512, rank=64, t_max=131072,
                topk=2048, window=0, layout=J.LAYOUT_MLA, scale=576 ** -0.5)
    base.update(kw)
    return _desc(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(), 0),
    (dict(rank=32), 0),
    (dict(n_q_heads=64), 0),
    (dict(reduce=J.REDUCE_MEAN), 0),
    (dict(n_kv_heads=2, n_q_heads=128), -1),  # one latent row per token
    (dict(d_v=640), -1),                      # the value is a prefix of the row
    (dict(rank=16), -2),
    (dict(n_q_heads=96), -2),
    (dict(d_k=512, d_v=448), -2),
    (dict(kv_dtype=J.F32, kp_dtype=J.F32), -2),
    (dict(kp_dtype=J.F32), -2),
    (dict(kp_dtype=J.FP8_E4M3), -2),          # MLA keeps bf16 projected keys
])
def test_mla_descriptor_validation(kw, status):
    for op in (J.OP_DECODE, J.OP_SCORE, J.OP_ATTN, J.OP_DENSE, 0):
        assert J.check_desc(_mla(**kw), op) == status, op


def test_mla_workspace_holds_query_fragments_and_partials():
    d = _mla()
    # projected-query fragments: B x (Hq/16 M-tiles) x (r/32 steps) x (hi, lo) x 1 KiB
    frag = 8 * 8 * 2 * 2 * 1024
    assert J.workspace_bytes(d, J.OP_SCORE) >= frag
    assert J.workspace_bytes(_mla(reduce=J.REDUCE_MEAN), J.OP_SCORE) < J.workspace_bytes(d, J.OP_SCORE)
    # attention partials: fp32 [B][chunks][Hq][512] for at least one chunk
    assert J.workspace_bytes(d, J.OP_ATTN) >= 8 * 128 * 512 * 4
    assert J.workspace_bytes(d, J.OP_DECODE) > J.workspace_bytes(d, J.OP_SCORE) + J.workspace_bytes(d, J.OP_ATTN)


def test_mla_entry_points_accept_null_v_cache_and_need_a_score_workspace():
    lib = J.lib()
    d = _mla().c()
    p = _fake(12)
    null = None
    # MLA scoring needs the workspace (the projected-query fragments)
    assert lib.jssa_score(d, *p[:5], null, 0, null) == -3
    assert lib.jssa_score(d, *p[:5], ctypes.c_void_p(4096), 64, null) == -3
    # v_cache is unused for MLA: a NULL v_cache passes the pointer checks and
    # the call fails on the missing workspace instead
    assert lib.jssa_indexed_attn(d, p[0], p[1], null, p[2], p[3], p[4], null, null, 0, null) == -3
    assert lib.jssa_dense_decode(d, p[0], p[1], null, p[2], p[3], null, null, 0, null) == -3
    assert lib.jssa_decode(d, *p[:4], null, p[4], p[5], null, null, null, null, 0, null) == -3
    # GQA still requires v_cache
    g = _desc().c()
    assert lib.jssa_dense_decode(g, p[0], p[1], null, p[2], p[3], null, null, 0, null) == -1


def test_static_decode_step_rejects_before_touching_the_gpu():
    """jssa_decode_step_static validates like jssa_decode_step, then rejects
    descriptors without a fused build and calls whose intermediates exceed its
    static scratch, all on the host."""
    lib = J.lib()
    p = _fake(13)
    null = None
    d = _desc().c()
    assert lib.jssa_decode_step_static(None, *p, null) == -1
    assert lib.jssa_decode_step_static(d, null, *p[1:], null) == -1          # k_new missing
    assert lib.jssa_decode_step_static(d, p[0], null, *p[2:], null) == -1    # GQA: v_new missing
    assert lib.jssa_decode_step_static(d, ctypes.c_void_p(4096 + 2), *p[1:], null) == -4
    assert lib.jssa_decode_step_static(_desc(n_q_heads=16).c(), *p, null) == -2  # G = 2 in bf16: staged shape
    assert lib.jssa_decode_step_static(_mla().c(), *p, null) == -2
    assert lib.jssa_decode_step_static(_desc(batch=64, t_max=1 << 20).c(), *p, null) == -6  # 4 GiB of slots
    assert lib.jssa_decode_step_static(_desc(batch=2048, n_kv_heads=8).c(), *p, null) == -6  # > 8192 rows
    assert lib.jssa_status_str(-6) == b"JSSA_ERR_TOO_LARGE"
