"""GPU parity on the selection paths that only large launches reach.

* More rows than scan workgroups.  The decode's scan normally gives every
  (sequence, KV head) row its own score workgroups, in proportion to the
  row's length.  With more rows than the device holds resident scan
  workgroups (1024 rows here), the rows' samples run in a launch of their
  own and the score work is split into equal contiguous ranges of the rows'
  tiles laid end to end, so ranges start and end inside rows.  The step's
  new token sits in the last candidate tile of every sequence.  The library's
  range-split counter proves the path ran.
* Cut in global memory.  With k = 16384 of 65536 candidates the sampled
  threshold passes about 21,000 tokens, more than the 16,384 the selection
  holds in shared memory, so the exact k-th key and tie cut run over the
  candidate slots in global memory (the library counts these rows), also after
  an exact re-selection (the sampled threshold admitted fewer than k tokens)
  and with crowded bins of equal keys.
* Every token a candidate.  A budget so close to the context (k = 30000 of
  32768) that the sample cannot bound it: the threshold stays open, each
  score tile keeps all its tokens and the selection reads the row's slots as
  one run (in shared memory up to 16,384, the rest in place).

Checks: the oracle on the same stored projected keys (set rule within 1e-4 of
the k-th score, attention within 2e-3 relative L2), and the stand-alone entry
points score -> top-k -> indexed attention on the same inputs (bit-identical
index lists: both are exact on the same fp32 scores)."""
import numpy as np
import pytest
import torch

import token_level_sparse_dim_amd as J
from oracle import jssa_oracle as O
from synth import WORKLOADS, generate, scaled, to_bf16_bits

from _gpu_helpers import check_sets_within_tolerance, desc_for, oracle_kp, rel_l2, to_dev, to_host

pytestmark = pytest.mark.gpu

MANY = scaled(WORKLOADS["hybrid_ragged"], batch=128, t_max=12000, t_min=9000, topk=1024)
GLOBAL = scaled(WORKLOADS["ctx128k"], batch=2, t_max=65536, topk=16384)
OPEN = scaled(WORKLOADS["ctx128k"], batch=2, t_max=32768, topk=30000)
_CACHE = {}


def _inputs(w):
    if w not in _CACHE:
        _CACHE[w] = generate(w)
    return _CACHE[w]


def _status(ws):
    return to_host(J.workspace_status(ws, clear=False))


def _decode(desc, w, dev_in, kp):
    out = torch.empty((w.batch, w.n_q_heads, w.d_v), device="cuda")
    lse = torch.empty((w.batch, w.n_q_heads), device="cuda")
    idx = torch.full((w.batch, w.n_kv_heads, w.topk + w.window), -1, dtype=torch.int32, device="cuda")
    n_sel = torch.zeros((w.batch, w.n_kv_heads), dtype=torch.int32, device="cuda")
    ws = J.workspace(desc, J.OP_DECODE)
    J.decode(desc, dev_in["q"], dev_in["P"], kp, dev_in["k_cache"], dev_in["v_cache"], dev_in["seq_lens"],
             out, lse, ws, idx_out=idx, n_sel_out=n_sel)
    torch.cuda.synchronize()
    return to_host(out), to_host(lse), to_host(idx), to_host(n_sel), ws


def _composed(desc, w, dev_in, kp):
    scores = torch.empty((w.batch, w.n_kv_heads, w.t_max), device="cuda")
    J.score(desc, dev_in["q"], dev_in["P"], kp, dev_in["seq_lens"], scores)
    idx = torch.full((w.batch, w.n_kv_heads, w.topk + w.window), -1, dtype=torch.int32, device="cuda")
    n_sel = torch.zeros((w.batch, w.n_kv_heads), dtype=torch.int32, device="cuda")
    J.topk(desc, scores, dev_in["seq_lens"], idx, n_sel, J.workspace(desc, J.OP_TOPK))
    out = torch.empty((w.batch, w.n_q_heads, w.d_v), device="cuda")
    J.indexed_attn(desc, dev_in["q"], dev_in["k_cache"], dev_in["v_cache"], idx, n_sel, out, None,
                   J.workspace(desc, J.OP_ATTN))
    torch.cuda.synchronize()
    return to_host(out), to_host(idx), to_host(n_sel), to_host(scores)


def _dev(inp):
    return {k: to_dev(inp[k]) for k in ("q", "P", "k_cache", "v_cache", "seq_lens")}


def test_more_rows_than_scan_workgroups_with_new_tokens():
    w = MANY
    inp = _inputs(w)
    desc = desc_for(w)
    B, Hkv, T, r, G = w.batch, w.n_kv_heads, w.t_max, w.rank, w.group
    L = inp["seq_lens"]
    assert (L - w.window > 8192).all()  # every row takes a sampled threshold
    d = _dev(inp)
    kp = torch.empty((B, Hkv, T, r), dtype=torch.bfloat16, device="cuda")
    J.append_projection(desc, T, torch.zeros(B, dtype=torch.int32, device="cuda"), d["P"], d["k_cache"], kp)
    samples = [(0, 0), (37, 3), (90, 5), (127, 7)]
    for b, h in samples:  # the oracle scores its own projection of the sampled rows
        n = int(L[b])
        kp[b, h, :n] = to_dev(O.project_keys(inp["k_cache"][b:b + 1, :n, h:h + 1], inp["P"][h:h + 1],
                                             np.array([n]), "bf16")[0][0, 0])
    # the step's new token at the last candidate position of every sequence
    rng = np.random.default_rng(5)
    kn = to_bf16_bits(rng.standard_normal((B, 1, Hkv, w.d_k)).astype(np.float32))
    vn = to_bf16_bits(rng.standard_normal((B, 1, Hkv, w.d_v)).astype(np.float32))
    pos = (L - w.window - 1).astype(np.int32)
    out = torch.empty((B, w.n_q_heads, w.d_v), device="cuda")
    lse = torch.empty((B, w.n_q_heads), device="cuda")
    idx = torch.full((B, Hkv, w.topk + w.window), -1, dtype=torch.int32, device="cuda")
    n_sel = torch.zeros((B, Hkv), dtype=torch.int32, device="cuda")
    ws = J.workspace(desc, J.OP_DECODE)
    J.decode_step(desc, to_dev(kn), to_dev(vn), to_dev(pos), d["q"], d["P"], kp, d["k_cache"], d["v_cache"],
                  d["seq_lens"], out, lse, ws, idx_out=idx, n_sel_out=n_sel)
    torch.cuda.synchronize()
    st = _status(ws)
    assert st[J.STATUS_RANGE_SPLIT] == 1, st  # the score work was split into ranges across rows
    gi, gn, go, gl = to_host(idx), to_host(n_sel), to_host(out), to_host(lse)
    assert np.isfinite(go).all() and np.isfinite(gl).all()
    # every row: the stand-alone entry points on the updated caches select the same lists
    o2, i2, n2, s32 = _composed(desc, w, d, kp)
    assert np.array_equal(gn, n2) and np.array_equal(gi, i2)
    assert rel_l2(go, o2) <= 1e-5
    # sampled rows: the oracle, with the new token in its caches
    k_host, v_host = inp["k_cache"].copy(), inp["v_cache"].copy()
    for b in range(B):
        k_host[b, pos[b]] = kn[b, 0]
        v_host[b, pos[b]] = vn[b, 0]
    for b, h in samples:
        n = int(L[b])
        kp_row = np.zeros((1, 1, T, r), np.uint16)
        kp_row[0, 0, :n] = to_host(kp[b, h, :n])  # the oracle's rows plus the GPU's appended row
        new = O.project_keys(kn[b:b + 1, :, h:h + 1], inp["P"][h:h + 1], np.array([1]), "bf16")[1][0, 0, 0]
        got = O.to_f64(kp_row[0, 0, pos[b]])
        bound = np.abs(O.to_f64(kn[b, 0, h])) @ np.abs(inp["P"][h].astype(np.float64)) * (1.01 * w.d_k * 2.0 ** -24)
        assert (np.abs(got - new) <= bound + np.ldexp(1.0, np.frexp(np.maximum(np.abs(got), np.abs(new)))[1] - 9)).all()
        hs = slice(h * G, (h + 1) * G)
        s64, n_cand = O.subspace_scores(inp["q"][b:b + 1, hs], inp["P"][h:h + 1], kp_row, L[b:b + 1], w.window)
        check_sets_within_tolerance(gi[b:b + 1, h:h + 1], gn[b:b + 1, h:h + 1], s64, n_cand, L[b:b + 1],
                                    w.topk, w.window)
        ref, ref_lse = O.attention(inp["q"][b:b + 1, hs], k_host[b:b + 1, :, h:h + 1], v_host[b:b + 1, :, h:h + 1],
                                   gi[b:b + 1, h:h + 1], gn[b:b + 1, h:h + 1], w.scale)
        assert rel_l2(go[b:b + 1, hs], ref) <= 2e-3, (b, h)
        assert np.abs(gl[b:b + 1, hs] - ref_lse).max() <= 1e-4 * max(1.0, np.abs(ref_lse).max())


@pytest.mark.parametrize("reduce", [J.REDUCE_MAX, J.REDUCE_MEAN], ids=["max", "mean"])
def test_global_cut_matches_oracle_and_composed(reduce):
    w = GLOBAL
    inp = _inputs(w)
    desc = desc_for(w, reduce=reduce)
    kp_h = oracle_kp(inp, desc)
    d = _dev(inp)
    kp = to_dev(kp_h)
    o1, l1, i1, n1, ws = _decode(desc, w, d, kp)
    assert _status(ws)[J.STATUS_GLOBAL_CUT] == w.batch * w.n_kv_heads  # every row took the global cut
    o2, i2, n2, _ = _composed(desc, w, d, kp)
    assert np.array_equal(n1, n2) and np.array_equal(i1, i2)
    assert rel_l2(o1, o2) <= 1e-5
    s64, n_cand = O.subspace_scores(inp["q"], inp["P"], kp_h, inp["seq_lens"], w.window,
                                    "max" if reduce == J.REDUCE_MAX else "mean")
    check_sets_within_tolerance(i1, n1, s64, n_cand, inp["seq_lens"], w.topk, w.window)
    ref, ref_lse = O.attention(inp["q"], inp["k_cache"], inp["v_cache"], i1, n1, w.scale)
    assert rel_l2(o1, ref) <= 2e-3
    assert np.abs(l1 - ref_lse).max() <= 1e-4 * max(1.0, np.abs(ref_lse).max())


@pytest.mark.parametrize("n_groups", [5, 60])
def test_global_cut_heavy_ties(n_groups):
    """Projected keys drawn from a few distinct rows: large groups of equal
    scores, the k-th inside one.  The selection is the oracle's full-sort top-k
    of the GPU's own fp32 scores, bit for bit."""
    w = GLOBAL
    inp = _inputs(w)
    desc = desc_for(w)
    kp_h = oracle_kp(inp, desc).copy()
    B, Hkv, T, _ = kp_h.shape
    rng = np.random.default_rng(31 + n_groups)
    for b in range(B):
        for h in range(Hkv):
            rows = kp_h[b, h, rng.choice(T, n_groups, replace=False)].copy()
            kp_h[b, h] = rows[rng.integers(0, n_groups, T)]
    d = _dev(inp)
    kp = to_dev(kp_h)
    o1, _, i1, n1, ws = _decode(desc, w, d, kp)
    assert _status(ws)[J.STATUS_GLOBAL_CUT] >= 1
    o2, i2, n2, s32 = _composed(desc, w, d, kp)
    assert np.array_equal(n1, n2) and np.array_equal(i1, i2)
    ref_idx, ref_n = O.topk_select(s32.astype(np.float64), inp["seq_lens"], w.topk, w.window)
    assert np.array_equal(ref_n, n1)
    for b in range(B):
        for h in range(Hkv):
            n = int(ref_n[b, h])
            assert np.array_equal(np.sort(ref_idx[b, h, :n]), i1[b, h, :n]), (b, h)
    ref, _ = O.attention(inp["q"], inp["k_cache"], inp["v_cache"], i1, n1, w.scale)
    assert rel_l2(o1, ref) <= 2e-3


def test_global_cut_after_exact_reselection():
    """Large scores planted on the token grid the threshold sample reads: the
    sample sees only them, its threshold admits fewer than k tokens, the row is
    re-selected exactly, and the exact candidates (every key in or above the
    k-th key's top radix bin) exceed shared memory."""
    w = GLOBAL
    inp = _inputs(w)
    desc = desc_for(w)
    kp_h = oracle_kp(inp, desc).copy()
    qp = O.project_query(inp["q"], inp["P"], w.n_kv_heads)
    s64, _ = O.subspace_scores(inp["q"], inp["P"], kp_h, inp["seq_lens"], w.window)
    smax = np.nanmax(np.abs(s64))
    rng = np.random.default_rng(13)
    G = w.group
    for b in range(w.batch):
        n_cand = int(inp["seq_lens"][b]) - w.window
        for h in range(w.n_kv_heads):
            v = qp[b, h * G]
            grid = np.arange(0, n_cand, n_cand // 1024)
            rows = (3.0 * smax / (v @ v)) * v[None, :] * (1.0 + 0.05 * rng.random((grid.size, 1)))
            kp_h[b, h, grid] = O.round_to_bf16_bits(rows)
    d = _dev(inp)
    kp = to_dev(kp_h)
    o1, _, i1, n1, ws = _decode(desc, w, d, kp)
    st = _status(ws)
    assert st[J.STATUS_EXACT_REDO] >= 1 and st[J.STATUS_GLOBAL_CUT] >= 1, st
    _, i2, n2, _ = _composed(desc, w, d, kp)
    assert np.array_equal(n1, n2) and np.array_equal(i1, i2)
    s64, n_cand = O.subspace_scores(inp["q"], inp["P"], kp_h, inp["seq_lens"], w.window)
    check_sets_within_tolerance(i1, n1, s64, n_cand, inp["seq_lens"], w.topk, w.window)
    ref, _ = O.attention(inp["q"], inp["k_cache"], inp["v_cache"], i1, n1, w.scale)
    assert rel_l2(o1, ref) <= 2e-3


def test_open_threshold_every_token_a_candidate():
    w = OPEN
    inp = _inputs(w)
    desc = desc_for(w)
    kp_h = oracle_kp(inp, desc)
    d = _dev(inp)
    kp = to_dev(kp_h)
    o1, l1, i1, n1, ws = _decode(desc, w, d, kp)
    assert _status(ws)[J.STATUS_GLOBAL_CUT] == w.batch * w.n_kv_heads  # 32768 candidates per row
    o2, i2, n2, _ = _composed(desc, w, d, kp)
    assert np.array_equal(n1, n2) and np.array_equal(i1, i2)
    assert rel_l2(o1, o2) <= 1e-5
    s64, n_cand = O.subspace_scores(inp["q"], inp["P"], kp_h, inp["seq_lens"], w.window)
    check_sets_within_tolerance(i1, n1, s64, n_cand, inp["seq_lens"], w.topk, w.window)
    ref, ref_lse = O.attention(inp["q"], inp["k_cache"], inp["v_cache"], i1, n1, w.scale)
    assert rel_l2(o1, ref) <= 2e-3
    assert np.abs(l1 - ref_lse).max() <= 1e-4 * max(1.0, np.abs(ref_lse).max())
