"""GPU tests of the decode step (a scan launch: sampled candidate threshold and
score scan; a resolve + attention launch) against the oracle and against the
composition of the stand-alone entry points (score -> top-k -> indexed
attention) on the same inputs.

The scan scores with the stand-alone score kernel's arithmetic and both
selections are exact by key with ties to the lower index, so the index lists
must be bit-identical; the attention outputs differ only by the chunking of
the softmax sums (fp32)."""
import numpy as np
import pytest
import torch

import token_level_sparse_dim_amd as J
from oracle import jssa_oracle as O
from synth import WORKLOADS, generate, scaled

from _gpu_helpers import (check_sets_within_tolerance, desc_for, oracle_kp, rel_l2, to_dev, to_host)

pytestmark = pytest.mark.gpu

CASES = {
    "tiny": WORKLOADS["tiny"],
    "llama": scaled(WORKLOADS["llama8b_32k"], batch=2, t_max=10000, topk=512),
    "128k": scaled(WORKLOADS["ctx128k"], batch=1, t_max=20000, topk=2048),
    "hybrid": scaled(WORKLOADS["hybrid_ragged"], batch=3, t_max=12000, t_min=3000, topk=256),
    "g1r64": scaled(WORKLOADS["llama8b_32k"], batch=1, n_q_heads=4, n_kv_heads=4, rank=64, t_max=6000,
                    topk=100, n_needles=8),
    "g2f32": scaled(WORKLOADS["tiny"], batch=2, n_q_heads=4, n_kv_heads=2, d_k=128, d_v=128, rank=32,
                    t_max=4500, topk=200, window=64),
    "d64bf16": scaled(WORKLOADS["llama8b_32k"], batch=2, d_k=64, d_v=64, rank=16, t_max=7000, topk=300),
}
_CACHE = {}


def inputs(w):
    if w not in _CACHE:
        _CACHE[w] = generate(w)
    return _CACHE[w]


def _run(desc, inp, kp, w, profiled):
    out = torch.empty((w.batch, w.n_q_heads, w.d_v), device="cuda")
    lse = torch.empty((w.batch, w.n_q_heads), device="cuda")
    idx = torch.full((w.batch, w.n_kv_heads, w.topk + w.window), -1, dtype=torch.int32, device="cuda")
    n_sel = torch.zeros((w.batch, w.n_kv_heads), dtype=torch.int32, device="cuda")
    ws = J.workspace(desc, J.OP_DECODE)
    args = (to_dev(inp["q"]), to_dev(inp["P"]), to_dev(kp), to_dev(inp["k_cache"]), to_dev(inp["v_cache"]),
            to_dev(inp["seq_lens"]))
    if profiled:
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        J.decode_profiled(desc, *args, out, lse, ws, ev, idx_out=idx, n_sel_out=n_sel)
    else:
        J.decode(desc, *args, out, lse, ws, idx_out=idx, n_sel_out=n_sel)
    torch.cuda.synchronize()
    return to_host(out), to_host(lse), to_host(idx), to_host(n_sel), ws


def _composed(desc, inp, kp, w):
    """score -> top-k -> indexed attention through the stand-alone entry points."""
    q, P, K, V, seq = (to_dev(inp[k]) for k in ("q", "P", "k_cache", "v_cache", "seq_lens"))
    scores = torch.empty((w.batch, w.n_kv_heads, w.t_max), device="cuda")
    J.score(desc, q, P, to_dev(kp), seq, scores)
    idx = torch.full((w.batch, w.n_kv_heads, w.topk + w.window), -1, dtype=torch.int32, device="cuda")
    n_sel = torch.zeros((w.batch, w.n_kv_heads), dtype=torch.int32, device="cuda")
    J.topk(desc, scores, seq, idx, n_sel, J.workspace(desc, J.OP_TOPK))
    out = torch.empty((w.batch, w.n_q_heads, w.d_v), device="cuda")
    lse = torch.empty((w.batch, w.n_q_heads), device="cuda")
    J.indexed_attn(desc, q, K, V, idx, n_sel, out, lse, J.workspace(desc, J.OP_ATTN))
    torch.cuda.synchronize()
    return to_host(out), to_host(lse), to_host(idx), to_host(n_sel)


def _fallbacks(ws):
    """Rows the decode re-selected exactly because the sampled threshold
    admitted fewer than k tokens (the library's diagnostic count, read without
    clearing it)."""
    return int(J.workspace_status(ws, clear=False).cpu()[J.STATUS_EXACT_REDO])


@pytest.mark.parametrize("reduce", [J.REDUCE_MAX, J.REDUCE_MEAN], ids=["max", "mean"])
@pytest.mark.parametrize("name", list(CASES))
def test_decode_matches_composed_entry_points(name, reduce):
    w = CASES[name]
    inp = inputs(w)
    desc = desc_for(w, reduce=reduce)
    kp = oracle_kp(inp, desc)
    o1, l1, i1, n1, _ = _run(desc, inp, kp, w, profiled=False)
    o2, l2, i2, n2 = _composed(desc, inp, kp, w)
    assert np.array_equal(n1, n2)
    assert np.array_equal(i1, i2)
    assert rel_l2(o1, o2) <= 1e-5
    fin = np.isfinite(l2)
    assert np.array_equal(fin, np.isfinite(l1))
    assert np.abs(l1[fin] - l2[fin]).max(initial=0.0) <= 1e-5 * max(1.0, np.abs(l2[fin]).max(initial=0.0))
    # the stage-event variant runs the same launches
    o3, _, i3, n3, _ = _run(desc, inp, kp, w, profiled=True)
    assert np.array_equal(i3, i1) and np.array_equal(n3, n1) and np.array_equal(o3, o1)
    # and the selection is the oracle's within the set rule
    s64, n_cand = O.subspace_scores(inp["q"], inp["P"], kp, inp["seq_lens"], w.window,
                                    "max" if reduce == J.REDUCE_MAX else "mean")
    check_sets_within_tolerance(i1, n1, s64, n_cand, inp["seq_lens"], w.topk, w.window)


def test_sample_threshold_fallback_is_exact():
    """Projected keys whose largest scores sit exactly on the token grid the
    threshold sample reads (every (n_cand // 1024)-th token for bf16 rank-32
    keys, whose sample is one 1024-token tile): the sample then sees only the
    top of the distribution, its threshold admits fewer than k tokens, and the
    row must be re-selected exactly."""
    w = CASES["llama"]
    inp = inputs(w)
    desc = desc_for(w)
    kp = oracle_kp(inp, desc).copy()  # [B, Hkv, T, r] bf16 bits
    qp = O.project_query(inp["q"], inp["P"], w.n_kv_heads)  # [B, Hq, r] fp64
    s64, _ = O.subspace_scores(inp["q"], inp["P"], kp, inp["seq_lens"], w.window)
    smax = np.nanmax(np.abs(s64))
    rng = np.random.default_rng(7)
    G = w.group
    for b in range(w.batch):
        n_cand = int(inp["seq_lens"][b]) - w.window
        assert n_cand > 8192  # the sampled path (fewer candidates are all kept)
        for h in range(w.n_kv_heads):
            v = qp[b, h * G]
            grid = np.arange(0, n_cand, n_cand // 1024)
            rows = (3.0 * smax / (v @ v)) * v[None, :] * (1.0 + 0.05 * rng.random((grid.size, 1)))
            kp[b, h, grid] = O.round_to_bf16_bits(rows)
    o1, _, i1, n1, ws = _run(desc, inp, kp, w, profiled=False)
    assert _fallbacks(ws) >= 1
    s64, n_cand = O.subspace_scores(inp["q"], inp["P"], kp, inp["seq_lens"], w.window)
    check_sets_within_tolerance(i1, n1, s64, n_cand, inp["seq_lens"], w.topk, w.window)
    _, _, i2, n2 = _composed(desc, inp, kp, w)
    assert np.array_equal(i1, i2) and np.array_equal(n1, n2)
    ref, _ = O.attention(inp["q"], inp["k_cache"], inp["v_cache"], np.where(i1 < 0, 0, i1), n1, w.scale)
    assert rel_l2(o1, ref) <= 2e-3


def test_fused_repeated_calls_share_workspace():
    """Back-to-back calls with different sequence lengths on one workspace: the
    per-row flags and the queue are left clean by every call."""
    w = CASES["hybrid"]
    inp = inputs(w)
    desc = desc_for(w)
    kp = oracle_kp(inp, desc)
    ws = J.workspace(desc, J.OP_DECODE)
    q, P, K, V = (to_dev(inp[k]) for k in ("q", "P", "k_cache", "v_cache"))
    KP = to_dev(kp)
    for lens in ([12000, 5000, 3000], [3000, 12000, 4097], [1, 700, 12000]):
        seq = np.array(lens, np.int32)
        out = torch.empty((w.batch, w.n_q_heads, w.d_v), device="cuda")
        idx = torch.full((w.batch, w.n_kv_heads, w.topk + w.window), -1, dtype=torch.int32, device="cuda")
        n_sel = torch.zeros((w.batch, w.n_kv_heads), dtype=torch.int32, device="cuda")
        J.decode(desc, q, P, KP, K, V, to_dev(seq), out, None, ws, idx_out=idx, n_sel_out=n_sel)
        gi, gn = to_host(idx), to_host(n_sel)
        s64, n_cand = O.subspace_scores(inp["q"], inp["P"], kp, seq, w.window)
        check_sets_within_tolerance(gi, gn, s64, n_cand, seq, w.topk, w.window)
        ref, _ = O.attention(inp["q"], inp["k_cache"], inp["v_cache"], np.where(gi < 0, 0, gi), gn, w.scale)
        assert rel_l2(to_host(out), ref) <= 2e-3


@pytest.mark.parametrize("n_groups,topk", [(5, 512), (5, 2500), (60, 512), (400, 700)],
                         ids=["inside_top_group", "inside_second_group", "60_groups", "400_groups"])
def test_decode_heavy_ties(n_groups, topk):
    """Projected keys drawn from a few distinct rows, so the scores form large
    groups of bitwise-equal values and the k-th lies inside one: the bin of
    the cut is crowded, and ties go to the lower token index.  The decode must
    equal the composed entry points, and the oracle's full-sort top-k on the
    GPU's own fp32 scores (bit-exact selection on identical score arrays)."""
    base = CASES["llama"]
    w = scaled(base, topk=topk)
    inp = inputs(base)
    desc = desc_for(w)
    kp = oracle_kp(inp, desc).copy()  # [B, Hkv, T, r] bf16 bits
    B, Hkv, T, _ = kp.shape
    rng = np.random.default_rng(11 + n_groups)
    for b in range(B):
        for h in range(Hkv):
            rows = kp[b, h, rng.choice(T, n_groups, replace=False)].copy()
            kp[b, h] = rows[rng.integers(0, n_groups, T)]
    o1, _, i1, n1, ws = _run(desc, inp, kp, w, profiled=False)
    o2, _, i2, n2 = _composed(desc, inp, kp, w)
    assert np.array_equal(n1, n2) and np.array_equal(i1, i2)
    assert rel_l2(o1, o2) <= 1e-5
    scores = torch.empty((w.batch, w.n_kv_heads, w.t_max), device="cuda")
    J.score(desc, to_dev(inp["q"]), to_dev(inp["P"]), to_dev(kp), to_dev(inp["seq_lens"]), scores)
    s32 = to_host(scores).astype(np.float64)
    ref_idx, ref_n = O.topk_select(s32, inp["seq_lens"], w.topk, w.window)
    assert np.array_equal(ref_n, n1)
    for b in range(B):
        for h in range(Hkv):
            n = int(ref_n[b, h])
            assert np.array_equal(np.sort(ref_idx[b, h, :n]), i1[b, h, :n]), (b, h)
    ref, _ = O.attention(inp["q"], inp["k_cache"], inp["v_cache"], np.where(i1 < 0, 0, i1), n1, w.scale)
    assert rel_l2(o1, ref) <= 2e-3
