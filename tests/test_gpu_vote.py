"""GPU tests of the head-shared soft-voting selection (``jssa_vote_select``;
JSSA summary section E.3 compares it with per-KV-head sets): on the GPU's
own fp32 scores, the shared lists equal the oracle's top-k of its fp64 vote
of those scores within the set rule (a token may differ only if its vote is
within 1e-4 relative of the k-th vote), every KV head gets the same list in
``jssa_topk``'s format, and the indexed attention over it matches the
oracle."""
import numpy as np
import pytest
import torch

import token_level_sparse_dim_amd as J
from oracle import jssa_oracle as O
from synth import WORKLOADS, generate, scaled

from _gpu_helpers import check_sets_within_tolerance, desc_for, oracle_kp, rel_l2, to_dev, to_host

pytestmark = pytest.mark.gpu

CASES = {
    "128k": scaled(WORKLOADS["ctx128k"], batch=2, t_max=20000, topk=2048),
    "llama": scaled(WORKLOADS["llama8b_32k"], batch=3, t_max=9000, topk=512),
    "hybrid": scaled(WORKLOADS["hybrid_ragged"], batch=4, t_max=12000, t_min=300, topk=256),
    "g8": scaled(WORKLOADS["llama8b_32k"], batch=2, n_q_heads=16, n_kv_heads=2, d_k=64, d_v=64,
                 rank=16, t_max=5000, topk=300, key_rank=8, n_needles=8),
}
_CACHE = {}


def inputs(w):
    if w not in _CACHE:
        _CACHE[w] = generate(w)
    return _CACHE[w]


@pytest.mark.parametrize("name", list(CASES))
def test_vote_select_matches_oracle(name):
    w = CASES[name]
    inp = inputs(w)
    seq = inp["seq_lens"].copy()
    if name == "hybrid":
        seq[1] = 0        # an empty sequence
        seq[2] = w.window + 100  # fewer candidates than the budget: all selected
    desc = desc_for(w)
    kp = oracle_kp({**inp, "seq_lens": seq}, desc)
    q, P, K, V = (to_dev(inp[k]) for k in ("q", "P", "k_cache", "v_cache"))
    S = to_dev(seq)
    scores = torch.empty((w.batch, w.n_kv_heads, w.t_max), device="cuda")
    J.score(desc, q, P, to_dev(kp), S, scores)
    idx = torch.full((w.batch, w.n_kv_heads, w.topk + w.window), -1, dtype=torch.int32, device="cuda")
    n_sel = torch.full((w.batch, w.n_kv_heads), -5, dtype=torch.int32, device="cuda")
    ws = J.workspace(desc, J.OP_VOTE)
    J.vote_select(desc, scores, S, idx, n_sel, ws)
    torch.cuda.synchronize()
    gi, gn = to_host(idx), to_host(n_sel)
    s32 = to_host(scores).astype(np.float64)
    for b in range(w.batch):  # every head holds the sequence's one list
        assert (gn[b] == gn[b, 0]).all()
        for h in range(1, w.n_kv_heads):
            assert np.array_equal(gi[b, h, :gn[b, 0]], gi[b, 0, :gn[b, 0]])
    vote = O.soft_vote(s32, seq, w.window, w.scale)
    n_cand = np.maximum(seq.astype(np.int64) - w.window, 0)
    check_sets_within_tolerance(gi[:, :1], gn[:, :1], vote, n_cand, seq, w.topk, w.window)
    # a second call on the same workspace: the same lists
    idx2 = torch.full_like(idx, -1)
    n2 = torch.zeros_like(n_sel)
    J.vote_select(desc, scores, S, idx2, n2, ws)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(n2), gn)
    for b in range(w.batch):
        assert np.array_equal(to_host(idx2)[b, :, :gn[b, 0]], gi[b, :, :gn[b, 0]])
    # the indexed attention over the shared lists
    out = torch.empty((w.batch, w.n_q_heads, w.d_v), device="cuda")
    lse = torch.empty((w.batch, w.n_q_heads), device="cuda")
    J.indexed_attn(desc, q, K, V, idx, n_sel, out, lse, J.workspace(desc, J.OP_ATTN))
    torch.cuda.synchronize()
    ref, ref_lse = O.attention(inp["q"], inp["k_cache"], inp["v_cache"], np.where(gi < 0, 0, gi), gn, w.scale)
    tol = 1e-5 if w.dtype == "f32" else 2e-3
    assert rel_l2(to_host(out), ref) <= tol
    fin = np.isfinite(ref_lse)
    assert np.array_equal(np.isfinite(to_host(lse)), fin)
    lse_err = np.abs(to_host(lse)[fin] - ref_lse[fin]).max(initial=0)
    assert lse_err <= 1e-4 * max(1.0, np.abs(ref_lse[fin]).max(initial=0))


def test_vote_select_one_head_is_per_head_topk():
    """With one KV head the vote ranks tokens as the head's scores do, so the
    shared list is the per-head top-k of the same scores (up to fp32 votes
    that round equal next to the k-th: the set rule on the scores)."""
    w = scaled(WORKLOADS["llama8b_32k"], batch=2, n_q_heads=4, n_kv_heads=1, t_max=6000, topk=400)
    inp = inputs(w)
    desc = desc_for(w)
    kp = oracle_kp(inp, desc)
    S = to_dev(inp["seq_lens"])
    scores = torch.empty((w.batch, 1, w.t_max), device="cuda")
    J.score(desc, to_dev(inp["q"]), to_dev(inp["P"]), to_dev(kp), S, scores)
    shape = (w.batch, 1, w.topk + w.window)
    i1 = torch.full(shape, -1, dtype=torch.int32, device="cuda")
    n1 = torch.zeros((w.batch, 1), dtype=torch.int32, device="cuda")
    i2, n2 = torch.full_like(i1, -1), torch.zeros_like(n1)
    J.vote_select(desc, scores, S, i1, n1, J.workspace(desc, J.OP_VOTE))
    J.topk(desc, scores, S, i2, n2, J.workspace(desc, J.OP_TOPK))
    torch.cuda.synchronize()
    assert np.array_equal(to_host(n1), to_host(n2))
    s64 = to_host(scores).astype(np.float64)
    n_cand = np.maximum(inp["seq_lens"].astype(np.int64) - w.window, 0)
    for i in (to_host(i1), to_host(i2)):
        check_sets_within_tolerance(i, to_host(n1), s64, n_cand, inp["seq_lens"], w.topk, w.window)
