"""GPU parity: every entry point of the HIP library against the CPU oracle on the
same seeded inputs, at sizes that span several tiles with ragged tails.

Rules (from the build contract): selection on identical fp32 score arrays is
bit-exact; end to end, the selected sets may differ only on tokens whose fp64
score lies within 1e-4 (relative) of the k-th score; attention outputs are
within 1e-5 relative L2 for fp32 inputs and 2e-3 for bf16 inputs."""
import numpy as np
import pytest
import torch

import token_level_sparse_dim_amd as J
from oracle import jssa_oracle as O
from synth import WORKLOADS, generate, scaled

from _gpu_helpers import (check_sets_within_tolerance, desc_for, oracle_kp, rel_l2, to_dev, to_host)

pytestmark = pytest.mark.gpu

W_TINY = WORKLOADS["tiny"]
W_LLAMA = scaled(WORKLOADS["llama8b_32k"], batch=2, t_max=10000, topk=512)
W_128K = scaled(WORKLOADS["ctx128k"], batch=1, t_max=20000, topk=2048)
W_HYB = scaled(WORKLOADS["hybrid_ragged"], batch=3, t_max=12000, t_min=3000, topk=256)
W_G8 = scaled(WORKLOADS["llama8b_32k"], batch=2, n_q_heads=16, n_kv_heads=2, d_k=64, d_v=64,
              rank=16, t_max=5000, topk=300, key_rank=8, n_needles=8)
W_G1 = scaled(WORKLOADS["llama8b_32k"], batch=1, n_q_heads=4, n_kv_heads=4, rank=64, t_max=6000,
              topk=100, n_needles=8)
W_G2F = scaled(WORKLOADS["tiny"], batch=2, n_q_heads=4, n_kv_heads=2, d_k=128, d_v=128, rank=32,
               t_max=4500, topk=200, window=64)
GQA_CASES = [W_TINY, W_LLAMA, W_128K, W_HYB, W_G8, W_G1, W_G2F]
IDS = ["tiny", "llama", "128k", "hybrid", "g8d64", "g1r64", "g2f32"]

_CACHE = {}


def inputs(w):
    if w not in _CACHE:
        _CACHE[w] = generate(w)
    return _CACHE[w]


def att_tol(w):
    return 1e-5 if w.dtype == "f32" else 2e-3


# ----------------------------------------------------------------------------- append / projection
def _ulp_distance(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Distance in representable bf16 steps between two bf16 bit arrays."""
    def ordered(u):
        u = u.astype(np.int64)
        return np.where(u & 0x8000, -(u & 0x7FFF), u)
    return np.abs(ordered(a) - ordered(b))


def _check_projection(got, stored, exact, k_cache, P, w):
    """GPU projection = round(y) with y the fp32-accumulated K.P, so
    |y - exact| <= d * 2^-24 * sum_d |K_d P_di| (recursive summation bound) and
    |got - exact| <= that bound + half a step of the stored format."""
    absK = np.abs(O.to_f64(k_cache))
    bound = np.zeros_like(exact)
    for h in range(w.n_kv_heads):
        bound[:, h] = absK[:, :, h, :] @ np.abs(P[h].astype(np.float64))
    bound *= 1.01 * w.d_k * 2.0 ** -24
    g64 = O.to_f64(got)
    if w.dtype == "f32":
        assert (np.abs(g64 - exact) <= bound + 1e-30).all()
    else:
        half_step = np.ldexp(1.0, np.frexp(np.maximum(np.abs(g64), np.abs(exact)))[1] - 9)
        assert (np.abs(g64 - exact) <= bound + half_step).all()
        big = np.abs(exact) > 512 * bound  # rounding error well below one step
        assert _ulp_distance(got[big], stored[big]).max() <= 1


@pytest.mark.parametrize("w", [W_TINY, W_LLAMA, W_G8, W_G1], ids=["tiny", "llama", "g8d64", "g1r64"])
def test_projection_of_cached_rows(w):
    inp = inputs(w)
    desc = desc_for(w)
    k = to_dev(inp["k_cache"])
    kp = torch.zeros((w.batch, w.n_kv_heads, w.t_max, w.rank),
                     dtype=torch.float32 if w.dtype == "f32" else torch.bfloat16, device="cuda")
    pos = torch.zeros(w.batch, dtype=torch.int32, device="cuda")
    J.append_projection(desc, w.t_max, pos, to_dev(inp["P"]), k, kp)
    got = to_host(kp)
    stored, exact = O.project_keys(inp["k_cache"], inp["P"], np.full(w.batch, w.t_max), "bf16" if w.dtype == "bf16" else "f32")
    _check_projection(got, stored, exact, inp["k_cache"], inp["P"], w)
    if w.dtype == "bf16":
        # the oracle's correctly rounded value except next to a rounding boundary
        assert (got != stored).mean() < 1e-3


@pytest.mark.parametrize("w", [W_TINY, W_LLAMA], ids=["tiny", "llama"])
def test_append_new_rows(w):
    inp = inputs(w)
    desc = desc_for(w)
    rng = np.random.default_rng(3)
    k = to_dev(inp["k_cache"])
    v = to_dev(inp["v_cache"])
    kp = torch.zeros((w.batch, w.n_kv_heads, w.t_max, w.rank), dtype=k.dtype, device="cuda")
    n_new = 3
    pos_h = np.array([w.t_max - 5 - 7 * b for b in range(w.batch)], np.int32)
    kn = rng.standard_normal((w.batch, n_new, w.n_kv_heads, w.d_k)).astype(np.float32)
    vn = rng.standard_normal((w.batch, n_new, w.n_kv_heads, w.d_v)).astype(np.float32)
    if w.dtype == "bf16":
        from synth import to_bf16_bits
        kn, vn = to_bf16_bits(kn), to_bf16_bits(vn)
    J.append_kv(desc, to_dev(kn), to_dev(vn), to_dev(pos_h), to_dev(inp["P"]), k, v, kp)
    kc, vc, kpc = to_host(k), to_host(v), to_host(kp)
    ref_k, ref_v = inp["k_cache"].copy(), inp["v_cache"].copy()
    for b in range(w.batch):
        ref_k[b, pos_h[b]:pos_h[b] + n_new] = kn[b]
        ref_v[b, pos_h[b]:pos_h[b] + n_new] = vn[b]
    assert np.array_equal(kc, ref_k) and np.array_equal(vc, ref_v)
    stored, exact = O.project_keys(ref_k, inp["P"], np.full(w.batch, w.t_max), "bf16" if w.dtype == "bf16" else "f32")
    for b in range(w.batch):
        rows = slice(pos_h[b], pos_h[b] + n_new)
        _check_projection(kpc[b:b + 1, :, rows], stored[b:b + 1, :, rows], exact[b:b + 1, :, rows],
                          ref_k[b:b + 1, rows], inp["P"], w)
        # nothing else was projected
        mask = np.ones(w.t_max, bool)
        mask[rows] = False
        assert (kpc[b][:, mask] == 0).all()


# ----------------------------------------------------------------------------- scores
@pytest.mark.parametrize("reduce", [J.REDUCE_MAX, J.REDUCE_MEAN], ids=["max", "mean"])
@pytest.mark.parametrize("w", GQA_CASES, ids=IDS)
def test_scores_match_oracle(w, reduce):
    inp = inputs(w)
    desc = desc_for(w, reduce=reduce)
    kp = oracle_kp(inp, desc)
    scores = torch.full((w.batch, w.n_kv_heads, w.t_max), 12345.0, device="cuda")
    J.score(desc, to_dev(inp["q"]), to_dev(inp["P"]), to_dev(kp), to_dev(inp["seq_lens"]), scores)
    got = to_host(scores).astype(np.float64)
    s64, n_cand = O.subspace_scores(inp["q"], inp["P"], kp, inp["seq_lens"], w.window,
                                    "max" if reduce == J.REDUCE_MAX else "mean")
    # fp32 error bound: (d_k + r) * 2^-23 * max_g sum_i |qp|_i |kp_i|, |qp|_i <= sum_d |q_d P_di|
    q64, P64 = np.abs(O.to_f64(inp["q"])), np.abs(inp["P"].astype(np.float64))
    G = w.group
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            n = int(n_cand[b])
            aqp = q64[b, h * G:(h + 1) * G] @ P64[h]  # [G, r]
            bound = (np.abs(O.to_f64(kp[b, h, :n])) @ aqp.T).max(axis=1) * (w.d_k + w.rank) * 2.0 ** -23
            err = np.abs(got[b, h, :n] - s64[b, h, :n])
            assert (err <= bound + 1e-30).all(), (b, h, err.max(), bound[err.argmax()])
            assert (got[b, h, n:] == 12345.0).all(), "non-candidates must not be written"


# ----------------------------------------------------------------------------- top-k (bit-exact)
def _score_arrays(kind, B, H, T, rng):
    if kind == "gauss":
        return rng.standard_normal((B, H, T)).astype(np.float32)
    if kind == "few_values":  # heavy exact ties across the threshold
        return rng.integers(-3, 4, size=(B, H, T)).astype(np.float32)
    if kind == "all_equal":
        return np.full((B, H, T), 0.75, np.float32)
    if kind == "specials":
        s = rng.standard_normal((B, H, T)).astype(np.float32)
        m = rng.random((B, H, T))
        s[m < 0.05] = np.nan
        s[(m >= 0.05) & (m < 0.08)] = np.inf
        s[(m >= 0.08) & (m < 0.11)] = -np.inf
        s[(m >= 0.11) & (m < 0.2)] = 0.0
        s[(m >= 0.2) & (m < 0.3)] = -0.0
        return s
    if kind == "narrow":  # many distinct values inside one first-digit bin
        base = np.float32(1.5)
        return (base + rng.integers(0, 50000, size=(B, H, T)).astype(np.float32) * np.float32(2.0 ** -22)).astype(np.float32)
    if kind == "needles":
        s = rng.standard_normal((B, H, T)).astype(np.float32)
        s[..., ::97] = 9.0
        return s
    raise ValueError(kind)


TOPK_CASES = [
    # kind, T, k, W, seq_lens
    ("gauss", 9000, 100, 0, [9000, 5000]),
    ("gauss", 9000, 2048, 0, [9000, 4097]),
    ("gauss", 9000, 1, 0, [9000, 8191]),
    ("few_values", 9000, 777, 0, [9000, 9000]),
    ("few_values", 13000, 4000, 100, [13000, 6000]),
    ("all_equal", 9000, 3000, 0, [9000, 4096]),
    ("all_equal", 9000, 5, 7, [9000, 20]),
    ("specials", 9000, 1500, 0, [9000, 3333]),
    ("narrow", 12288, 5000, 0, [12288, 12000]),
    ("needles", 9000, 93, 16, [9000, 8800]),
    ("gauss", 9000, 9000, 0, [9000, 100]),      # k >= candidates: every candidate
    ("gauss", 9000, 0, 64, [9000, 30]),         # window only
    ("gauss", 9000, 300, 512, [9000, 512]),     # a sequence with no candidates
    ("gauss", 9000, 300, 0, [0, 7]),            # an empty sequence
]


@pytest.mark.parametrize("kind,T,k,W,lens", TOPK_CASES)
def test_topk_bit_exact(kind, T, k, W, lens):
    rng = np.random.default_rng(abs(hash((kind, T, k, W))) % 2**32)
    B, H = len(lens), 3
    s = _score_arrays(kind, B, H, T, rng)
    seq = np.array(lens, np.int32)
    desc = J.Desc(batch=B, n_q_heads=H, n_kv_heads=H, d_k=64, d_v=64, rank=16, t_max=T, topk=k,
                  window=W, kv_dtype=J.F32, kp_dtype=J.F32, scale=0.125)
    ws = J.workspace(desc, J.OP_TOPK)
    idx = torch.full((B, H, k + W), -7, dtype=torch.int32, device="cuda")
    n_sel = torch.zeros((B, H), dtype=torch.int32, device="cuda")
    ref_idx, ref_n = O.topk_select(s, seq, k, W)
    for rep in range(2):  # the workspace is reused: counters must come back zeroed
        J.topk(desc, to_dev(s), to_dev(seq), idx, n_sel, ws)
        gi, gn = to_host(idx), to_host(n_sel)
        assert np.array_equal(gn, ref_n)
        for b in range(B):
            for h in range(H):
                n = ref_n[b, h]
                assert np.array_equal(gi[b, h, :n], ref_idx[b, h, :n]), (rep, b, h)


# ----------------------------------------------------------------------------- attention
@pytest.mark.parametrize("out_dtype", [J.F32, J.BF16], ids=["out_f32", "out_bf16"])
@pytest.mark.parametrize("w", GQA_CASES, ids=IDS)
def test_indexed_attention_matches_oracle(w, out_dtype):
    inp = inputs(w)
    desc = desc_for(w, out_dtype=out_dtype)
    kp = oracle_kp(inp, desc)
    s64, _ = O.subspace_scores(inp["q"], inp["P"], kp, inp["seq_lens"], w.window)
    idx, n_sel = O.topk_select(s64, inp["seq_lens"], w.topk, w.window)
    out = torch.empty((w.batch, w.n_q_heads, w.d_v), dtype=torch.float32 if out_dtype == J.F32 else torch.bfloat16, device="cuda")
    lse = torch.empty((w.batch, w.n_q_heads), device="cuda")
    ws = J.workspace(desc, J.OP_ATTN)
    J.indexed_attn(desc, to_dev(inp["q"]), to_dev(inp["k_cache"]), to_dev(inp["v_cache"]),
                   to_dev(np.where(idx < 0, 0, idx).astype(np.int32)), to_dev(n_sel), out, lse, ws)
    ref, ref_lse = O.attention(inp["q"], inp["k_cache"], inp["v_cache"], idx, n_sel, w.scale)
    got = to_host(out)
    got = O.to_f64(got) if out_dtype == J.BF16 else got
    tol = att_tol(w) + (2.0 ** -8 if out_dtype == J.BF16 else 0.0)
    assert rel_l2(got, ref) <= tol
    assert np.abs(to_host(lse) - ref_lse).max() <= 1e-4 * max(1.0, np.abs(ref_lse).max())


@pytest.mark.parametrize("w", GQA_CASES, ids=IDS)
def test_dense_decode_matches_oracle(w):
    inp = inputs(w)
    desc = desc_for(w)
    out = torch.empty((w.batch, w.n_q_heads, w.d_v), device="cuda")
    lse = torch.empty((w.batch, w.n_q_heads), device="cuda")
    ws = J.workspace(desc, J.OP_DENSE)
    J.dense_decode(desc, to_dev(inp["q"]), to_dev(inp["k_cache"]), to_dev(inp["v_cache"]),
                   to_dev(inp["seq_lens"]), out, lse, ws)
    ref, ref_lse = O.dense_attention(inp["q"], inp["k_cache"], inp["v_cache"], inp["seq_lens"], w.scale)
    assert rel_l2(to_host(out), ref) <= att_tol(w)
    assert np.abs(to_host(lse) - ref_lse).max() <= 1e-4 * max(1.0, np.abs(ref_lse).max())


# ----------------------------------------------------------------------------- fused decode
@pytest.mark.parametrize("reduce", [J.REDUCE_MAX, J.REDUCE_MEAN], ids=["max", "mean"])
@pytest.mark.parametrize("w", GQA_CASES, ids=IDS)
def test_decode_end_to_end(w, reduce):
    inp = inputs(w)
    desc = desc_for(w, reduce=reduce)
    kp = oracle_kp(inp, desc)
    out = torch.empty((w.batch, w.n_q_heads, w.d_v), device="cuda")
    lse = torch.empty((w.batch, w.n_q_heads), device="cuda")
    idx = torch.full((w.batch, w.n_kv_heads, w.topk + w.window), -1, dtype=torch.int32, device="cuda")
    n_sel = torch.zeros((w.batch, w.n_kv_heads), dtype=torch.int32, device="cuda")
    ws = J.workspace(desc, J.OP_DECODE)
    args = (to_dev(inp["q"]), to_dev(inp["P"]), to_dev(kp), to_dev(inp["k_cache"]), to_dev(inp["v_cache"]),
            to_dev(inp["seq_lens"]))
    J.decode(desc, *args, out, lse, ws, idx_out=idx, n_sel_out=n_sel)
    gi, gn = to_host(idx), to_host(n_sel)
    s64, n_cand = O.subspace_scores(inp["q"], inp["P"], kp, inp["seq_lens"], w.window,
                                    "max" if reduce == J.REDUCE_MAX else "mean")
    check_sets_within_tolerance(gi, gn, s64, n_cand, inp["seq_lens"], w.topk, w.window)
    # attention on the GPU's own selection
    ref, ref_lse = O.attention(inp["q"], inp["k_cache"], inp["v_cache"], np.where(gi < 0, 0, gi), gn, w.scale)
    o1 = to_host(out).copy()
    assert rel_l2(o1, ref) <= att_tol(w)
    assert np.abs(to_host(lse) - ref_lse).max() <= 1e-4 * max(1.0, np.abs(ref_lse).max())
    # determinism: a second call (same workspace) is bitwise identical
    J.decode(desc, *args, out, lse, ws, idx_out=idx, n_sel_out=n_sel)
    assert np.array_equal(to_host(out), o1) and np.array_equal(to_host(idx), gi)


def test_decode_full_rank_basis_is_exact_attention_topk():
    """r = d with P = I: the subspace score is the exact max_g q_g.k, so the fused
    decode selects the exact-attention-logit top-k (set rule) and attends over it."""
    w = scaled(W_TINY, rank=64)
    inp = inputs(W_TINY)
    P = np.broadcast_to(np.eye(64, dtype=np.float32), (w.n_kv_heads, 64, 64)).copy()
    desc = desc_for(w)
    kp, _ = O.project_keys(inp["k_cache"], P, inp["seq_lens"], "f32")
    idx = torch.full((w.batch, w.n_kv_heads, w.topk), -1, dtype=torch.int32, device="cuda")
    n_sel = torch.zeros((w.batch, w.n_kv_heads), dtype=torch.int32, device="cuda")
    out = torch.empty((w.batch, w.n_q_heads, w.d_v), device="cuda")
    ws = J.workspace(desc, J.OP_DECODE)
    J.decode(desc, to_dev(inp["q"]), to_dev(P), to_dev(kp), to_dev(inp["k_cache"]),
             to_dev(inp["v_cache"]), to_dev(inp["seq_lens"]), out, None, ws, idx_out=idx, n_sel_out=n_sel)
    gi, gn = to_host(idx), to_host(n_sel)
    # exact logits q.k (no projection at all), max over each KV head's group
    q64, K64 = O.to_f64(inp["q"]), O.to_f64(inp["k_cache"])
    G = w.group
    exact = np.stack([np.max(K64[0, :, h, :] @ q64[0, h * G:(h + 1) * G].T, axis=1)
                      for h in range(w.n_kv_heads)])[None]
    check_sets_within_tolerance(gi, gn, exact, np.array([w.t_max]), inp["seq_lens"], w.topk, 0)
    ref, _ = O.attention(inp["q"], inp["k_cache"], inp["v_cache"], gi, gn, w.scale)
    assert rel_l2(to_host(out), ref) <= att_tol(w)


def test_decode_edge_lengths():
    """Empty sequence, a sequence inside the window, budget above the candidates."""
    w = scaled(W_HYB, batch=4, t_max=6000, t_min=None, topk=700, window=512)
    inp = inputs(scaled(w, t_min=3000))
    seq = np.array([0, 300, 1000, 6000], np.int32)
    desc = desc_for(w)
    kp = oracle_kp({**inp, "seq_lens": seq}, desc)
    out = torch.full((w.batch, w.n_q_heads, w.d_v), 7.0, device="cuda")
    lse = torch.empty((w.batch, w.n_q_heads), device="cuda")
    idx = torch.full((w.batch, w.n_kv_heads, w.topk + w.window), -1, dtype=torch.int32, device="cuda")
    n_sel = torch.zeros((w.batch, w.n_kv_heads), dtype=torch.int32, device="cuda")
    ws = J.workspace(desc, J.OP_DECODE)
    J.decode(desc, to_dev(inp["q"]), to_dev(inp["P"]), to_dev(kp), to_dev(inp["k_cache"]),
             to_dev(inp["v_cache"]), to_dev(seq), out, lse, ws, idx_out=idx, n_sel_out=n_sel)
    gi, gn = to_host(idx), to_host(n_sel)
    s64, n_cand = O.subspace_scores(inp["q"], inp["P"], kp, seq, w.window)
    assert gn[:, 0].tolist() == [0, 300, 1000, 1212]
    check_sets_within_tolerance(gi, gn, s64, n_cand, seq, w.topk, w.window)
    o = to_host(out)
    assert (o[0] == 0).all() and np.isneginf(to_host(lse)[0]).all()
    ref, _ = O.attention(inp["q"], inp["k_cache"], inp["v_cache"], np.where(gi < 0, 0, gi), gn, w.scale)
    assert rel_l2(o[1:], ref[1:]) <= att_tol(w)
