"""GPU parity of the MLA layout (one shared 576-wide latent row per token, the
value is its first 512 columns, one index set per sequence) against the CPU
oracle: scores, selection, indexed attention, the whole decode step and the
dense comparison path, on seeded inputs that span several score tiles,
attention chunks and sub-blocks with ragged tails.

Tolerances: scores within the bound of the arithmetic (projected query in fp32
entering the matrix-core product as two bf16 terms, fp32 accumulation);
selection on identical fp32 scores bit-exact; end-to-end sets by the 1e-4 rule;
attention within 2e-3 relative L2 (the bar for bf16 inputs) and, since q, K and
V enter the products exactly and the probabilities with about 16 bits, within
1e-4 as well."""
import numpy as np
import pytest
import torch

import token_level_sparse_dim_amd as J
from oracle import jssa_oracle as O
from synth import WORKLOADS, generate, scaled

from _gpu_helpers import (check_sets_within_tolerance, desc_for, oracle_kp, rel_l2, to_dev, to_host)

pytestmark = pytest.mark.gpu

W_BASE = WORKLOADS["mla"]
W_A = scaled(W_BASE, batch=2, t_max=6000, topk=512)
W_RAG = scaled(W_BASE, batch=3, t_max=7000, t_min=2000, topk=700, window=96)
W_H64 = scaled(W_BASE, batch=2, n_q_heads=64, rank=32, t_max=4100, topk=300, n_needles=16)
W_B8 = scaled(W_BASE, batch=8, t_max=3000, topk=1500)
CASES = [W_A, W_RAG, W_H64, W_B8]
IDS = ["h128r64", "ragged_window", "h64r32", "b8_multi_sub"]

_CACHE = {}


def inputs(w):
    if w not in _CACHE:
        _CACHE[w] = generate(w)
    return _CACHE[w]


def v_view(inp, w):
    """The oracle's value cache for MLA: a view of the first d_v columns of K."""
    return inp["k_cache"][..., :w.d_v]


def _attend_ref(inp, w, idx, n_sel):
    return O.attention(inp["q"], inp["k_cache"], v_view(inp, w), idx, n_sel, w.scale)


def _check_attention(out, lse, ref_out, ref_lse):
    assert rel_l2(out, ref_out) <= 2e-3
    assert rel_l2(out, ref_out) <= 1e-4, rel_l2(out, ref_out)
    fin = np.isfinite(ref_lse)
    assert np.array_equal(np.isfinite(lse), fin)
    assert np.abs(lse[fin] - ref_lse[fin]).max(initial=0) <= 1e-4 * max(1.0, np.abs(ref_lse[fin]).max(initial=0))


def _score_bound(inp, w, kp, n_cand, reduce):
    """|s_gpu - s64| bound per token: qp coordinates carry 2^-17 (hi + lo
    split) plus fp32 rounding of the projection and of the accumulation."""
    q64, P64 = np.abs(O.to_f64(inp["q"])), np.abs(inp["P"][0].astype(np.float64))
    bounds = []
    for b in range(w.batch):
        n = int(n_cand[b])
        kpa = np.abs(O.to_f64(kp[b, 0, :n]))
        if reduce == J.REDUCE_MAX:
            e = (kpa @ (q64[b] @ P64).T).max(axis=1)
            rel = 2.0 ** -16 + (w.d_k + w.rank) * 2.0 ** -23
        else:
            e = kpa @ (q64[b].mean(axis=0) @ P64)
            rel = 2.0 ** -16 + (w.n_q_heads + w.d_k + w.rank) * 2.0 ** -23
        bounds.append(e * rel)
    return bounds


@pytest.mark.parametrize("reduce", [J.REDUCE_MAX, J.REDUCE_MEAN], ids=["max", "mean"])
@pytest.mark.parametrize("w", CASES, ids=IDS)
def test_mla_scores_match_oracle(w, reduce):
    inp = inputs(w)
    desc = desc_for(w, reduce=reduce)
    kp = oracle_kp(inp, desc)
    scores = torch.full((w.batch, 1, w.t_max), 12345.0, device="cuda")
    ws = J.workspace(desc, J.OP_SCORE)
    J.score(desc, to_dev(inp["q"]), to_dev(inp["P"]), to_dev(kp), to_dev(inp["seq_lens"]), scores, ws)
    got = to_host(scores).astype(np.float64)
    s64, n_cand = O.subspace_scores(inp["q"], inp["P"], kp, inp["seq_lens"], w.window,
                                    "max" if reduce == J.REDUCE_MAX else "mean")
    for b, bound in enumerate(_score_bound(inp, w, kp, n_cand, reduce)):
        n = int(n_cand[b])
        err = np.abs(got[b, 0, :n] - s64[b, 0, :n])
        assert (err <= bound + 1e-30).all(), (b, err.max(), bound[err.argmax()])
        assert (got[b, 0, n:] == 12345.0).all(), "non-candidates must not be written"


@pytest.mark.parametrize("reduce", [J.REDUCE_MAX, J.REDUCE_MEAN], ids=["max", "mean"])
@pytest.mark.parametrize("w", CASES, ids=IDS)
def test_mla_decode_matches_oracle_and_composed_calls(w, reduce):
    inp = inputs(w)
    desc = desc_for(w, reduce=reduce)
    kp = oracle_kp(inp, desc)
    q, P, k, seq = to_dev(inp["q"]), to_dev(inp["P"]), to_dev(inp["k_cache"]), to_dev(inp["seq_lens"])
    kpd = to_dev(kp)
    n_max = w.topk + w.window
    out = torch.empty((w.batch, w.n_q_heads, w.d_v), device="cuda")
    lse = torch.empty((w.batch, w.n_q_heads), device="cuda")
    idx = torch.full((w.batch, 1, n_max), -7, dtype=torch.int32, device="cuda")
    n_sel = torch.empty((w.batch, 1), dtype=torch.int32, device="cuda")
    ws = J.workspace(desc, J.OP_DECODE)
    for _ in range(2):  # the workspace is reused: the second call must agree
        J.decode(desc, q, P, kpd, k, None, seq, out, lse, ws, idx_out=idx, n_sel_out=n_sel)
    torch.cuda.synchronize()
    g_idx, g_n = to_host(idx), to_host(n_sel)

    # the same selection as the stand-alone entry points on the same scores
    scores = torch.empty((w.batch, 1, w.t_max), device="cuda")
    J.score(desc, q, P, kpd, seq, scores, J.workspace(desc, J.OP_SCORE))
    idx2 = torch.full_like(idx, -7)
    n2 = torch.empty_like(n_sel)
    J.topk(desc, scores, seq, idx2, n2, J.workspace(desc, J.OP_TOPK))
    assert np.array_equal(to_host(n2), g_n)
    for b in range(w.batch):
        assert np.array_equal(to_host(idx2)[b, 0, :g_n[b, 0]], g_idx[b, 0, :g_n[b, 0]])

    # end to end against the oracle's selection rule
    s64, n_cand = O.subspace_scores(inp["q"], inp["P"], kp, inp["seq_lens"], w.window,
                                    "max" if reduce == J.REDUCE_MAX else "mean")
    check_sets_within_tolerance(g_idx, g_n, s64, n_cand, inp["seq_lens"], w.topk, w.window)

    # attention over the selected rows
    ref_out, ref_lse = _attend_ref(inp, w, g_idx, g_n)
    _check_attention(to_host(out), to_host(lse), ref_out, ref_lse)


@pytest.mark.parametrize("w", CASES, ids=IDS)
def test_mla_indexed_attention_matches_oracle(w):
    inp = inputs(w)
    desc = desc_for(w)
    n_max = w.topk + w.window
    rng = np.random.default_rng(11)
    # arbitrary (unsorted) index lists with one sequence attending over nothing
    idx = np.full((w.batch, 1, n_max), -1, np.int32)
    n_sel = np.zeros((w.batch, 1), np.int32)
    for b in range(w.batch):
        Tb = int(inp["seq_lens"][b])
        n = 0 if b == 1 else min(n_max, Tb) - (b % 3) * 17
        idx[b, 0, :n] = rng.choice(Tb, size=n, replace=False)
        n_sel[b, 0] = n
    out = torch.empty((w.batch, w.n_q_heads, w.d_v), device="cuda")
    lse = torch.empty((w.batch, w.n_q_heads), device="cuda")
    ws = J.workspace(desc, J.OP_ATTN)
    J.indexed_attn(desc, to_dev(inp["q"]), to_dev(inp["k_cache"]), None, to_dev(idx), to_dev(n_sel),
                   out, lse, ws)
    got, got_lse = to_host(out), to_host(lse)
    ref_out, ref_lse = _attend_ref(inp, w, idx, n_sel)
    _check_attention(got, got_lse, ref_out, ref_lse)
    assert (got[1] == 0).all() and np.isneginf(got_lse[1]).all()


@pytest.mark.parametrize("w", [W_A, W_RAG, W_B8], ids=["h128r64", "ragged_window", "b8_multi_sub"])
def test_mla_dense_matches_oracle(w):
    inp = inputs(w)
    desc = desc_for(w)
    out = torch.empty((w.batch, w.n_q_heads, w.d_v), device="cuda")
    lse = torch.empty((w.batch, w.n_q_heads), device="cuda")
    J.dense_decode(desc, to_dev(inp["q"]), to_dev(inp["k_cache"]), None, to_dev(inp["seq_lens"]), out, lse,
                   J.workspace(desc, J.OP_DENSE))
    ref_out, ref_lse = O.dense_attention(inp["q"], inp["k_cache"], v_view(inp, w), inp["seq_lens"], w.scale)
    _check_attention(to_host(out), to_host(lse), ref_out, ref_lse)


def test_mla_budget_covering_every_token_equals_dense():
    w = scaled(W_BASE, batch=2, t_max=2500, topk=2500)
    inp = inputs(w)
    desc = desc_for(w, out_dtype=J.BF16)
    kpd = to_dev(oracle_kp(inp, desc))
    q, P, k, seq = to_dev(inp["q"]), to_dev(inp["P"]), to_dev(inp["k_cache"]), to_dev(inp["seq_lens"])
    out = torch.empty((w.batch, w.n_q_heads, w.d_v), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.batch, w.n_q_heads), device="cuda")
    J.decode(desc, q, P, kpd, k, None, seq, out, lse, J.workspace(desc, J.OP_DECODE))
    ref_out, ref_lse = O.dense_attention(inp["q"], inp["k_cache"], v_view(inp, w), inp["seq_lens"], w.scale)
    got = O.to_f64(to_host(out))
    # a bf16 output adds at most half a bf16 step per element
    assert rel_l2(got, ref_out) <= 2e-3
    assert np.abs(to_host(lse) - ref_lse).max() <= 1e-4 * max(1.0, np.abs(ref_lse).max())


def test_mla_empty_and_short_sequences():
    w = scaled(W_BASE, batch=3, t_max=3000, topk=256, window=32)
    inp = dict(inputs(w))
    inp["seq_lens"] = np.array([0, 20, 3000], np.int32)  # empty; window only; full
    desc = desc_for(w)
    kp = O.project_keys(inp["k_cache"], inp["P"], inp["seq_lens"], "bf16")[0]
    out = torch.empty((w.batch, w.n_q_heads, w.d_v), device="cuda")
    lse = torch.empty((w.batch, w.n_q_heads), device="cuda")
    idx = torch.full((w.batch, 1, w.topk + w.window), -7, dtype=torch.int32, device="cuda")
    n_sel = torch.empty((w.batch, 1), dtype=torch.int32, device="cuda")
    J.decode(desc, to_dev(inp["q"]), to_dev(inp["P"]), to_dev(kp), to_dev(inp["k_cache"]), None,
             to_dev(inp["seq_lens"]), out, lse, J.workspace(desc, J.OP_DECODE), idx_out=idx, n_sel_out=n_sel)
    g_idx, g_n = to_host(idx), to_host(n_sel)
    assert g_n[:, 0].tolist() == [0, 20, 256 + 32]
    assert g_idx[1, 0, :20].tolist() == list(range(20))
    ref_out, ref_lse = _attend_ref(inp, w, g_idx, g_n)
    got, got_lse = to_host(out), to_host(lse)
    _check_attention(got, got_lse, ref_out, ref_lse)
    assert (got[0] == 0).all() and np.isneginf(got_lse[0]).all()


@pytest.mark.parametrize("n_new", [1, 3])
@pytest.mark.parametrize("w", [W_A, W_H64], ids=["r64", "r32"])
def test_mla_append_new_rows(w, n_new):
    """A step's new latent rows (the wide-row append: 1024 threads per row):
    the rows are copied into the cache, their keys projected within the fp32
    summation bound plus half a bf16 step of the exact product and equal to
    the oracle's rounding except next to a rounding boundary; nothing else is
    written."""
    from synth import to_bf16_bits
    inp = inputs(w)
    desc = desc_for(w)
    rng = np.random.default_rng(31 + n_new)
    k = to_dev(inp["k_cache"])
    kp = torch.zeros((w.batch, 1, w.t_max, w.rank), dtype=torch.bfloat16, device="cuda")
    pos = np.array([w.t_max - 4 - 5 * b for b in range(w.batch)], np.int32)
    kn = to_bf16_bits(rng.standard_normal((w.batch, n_new, 1, w.d_k)).astype(np.float32))
    J.append_kv(desc, to_dev(kn), None, to_dev(pos), to_dev(inp["P"]), k, None, kp)
    ref_k = inp["k_cache"].copy()
    for b in range(w.batch):
        ref_k[b, pos[b]:pos[b] + n_new] = kn[b]
    assert np.array_equal(to_host(k), ref_k)
    stored, exact = O.project_keys(ref_k, inp["P"], np.full(w.batch, w.t_max), "bf16")
    got = to_host(kp)
    absK = np.abs(O.to_f64(ref_k))
    for b in range(w.batch):
        rows = slice(pos[b], pos[b] + n_new)
        bound = (absK[b, rows, 0] @ np.abs(inp["P"][0].astype(np.float64))) * (1.01 * w.d_k * 2.0 ** -24)
        g64, ex = O.to_f64(got[b, 0, rows]), exact[b, 0, rows]
        half = np.ldexp(1.0, np.frexp(np.maximum(np.abs(g64), np.abs(ex)))[1] - 9)
        assert (np.abs(g64 - ex) <= bound + half).all()
        assert (got[b, 0, rows] != stored[b, 0, rows]).mean() <= 0.05
        mask = np.ones(w.t_max, bool)
        mask[rows] = False
        assert (got[b, 0, mask] == 0).all()
