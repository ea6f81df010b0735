"""GPU parity of the FP8 (E4M3) projected-key cache against the oracle and
against the bf16-key paths' own rules.

The pages keep the scoring cache in FP8 (JSSA summary appendix A.3; section
E.2: it halves the cache against BF16).  The projection rounds the
fp32-accumulated K.P once to E4M3 (nearest even, saturating); the scan widens
the codes to bf16 exactly and scores them on the matrix cores like bf16 keys.
So: the projection is within the fp32 summation bound plus half an E4M3 step
of the exact product and equals the oracle's code except next to a rounding
boundary; scores fed the oracle's codes are within the fp32 bound of the fp64
scores; selection and attention follow the same rules as for bf16 keys; the
fused decode equals the composed entry points bit for bit."""
import numpy as np
import pytest
import torch

import token_level_sparse_dim_amd as J
from oracle import jssa_oracle as O
from synth import WORKLOADS, generate, scaled, to_bf16_bits

from _gpu_helpers import check_sets_within_tolerance, desc_for, oracle_kp, rel_l2, to_dev, to_host

pytestmark = pytest.mark.gpu

FP8 = J.FP8_E4M3
CASES = {
    "128k": scaled(WORKLOADS["ctx128k"], batch=2, t_max=20000, topk=2048),
    "llama": scaled(WORKLOADS["llama8b_32k"], batch=2, t_max=10000, topk=512),
    "hybrid": scaled(WORKLOADS["hybrid_ragged"], batch=3, t_max=12000, t_min=3000, topk=256),
    "g1r64": scaled(WORKLOADS["llama8b_32k"], batch=2, n_q_heads=4, n_kv_heads=4, rank=64, t_max=6000,
                    topk=100, n_needles=8),
    "g2": scaled(WORKLOADS["llama8b_32k"], batch=2, n_q_heads=16, n_kv_heads=8, t_max=5000,
                 topk=128),  # G = 2: the staged launches
    "g8": scaled(WORKLOADS["llama8b_32k"], batch=1, n_q_heads=16, n_kv_heads=2, t_max=7000, topk=300),
}
_CACHE = {}


def inputs(w):
    if w not in _CACHE:
        _CACHE[w] = generate(w)
    return _CACHE[w]


def fdesc(w, **kw):
    return desc_for(w, kp_dtype=FP8, **kw)


def _kp_empty(w):
    return torch.zeros((w.batch, w.n_kv_heads, w.t_max, w.rank), dtype=torch.uint8, device="cuda")


def _e4m3_half_step(x):
    """Half the E4M3 spacing around |x| (spacing 2^(e-3), e >= -6)."""
    e = np.maximum(np.frexp(np.abs(x))[1] - 1, -6)
    return np.ldexp(1.0, e - 4)


def _check_projection_fp8(got, stored, exact, k_rows, P, w):
    """got = round_e4m3(y), y the fp32-accumulated K.P: |got - exact| <= the
    summation bound + half a step (exact clamped to +-448: saturation); got ==
    the oracle's code except where the exact value lies within the bound of a
    rounding boundary."""
    absK = np.abs(O.to_f64(k_rows))
    bound = np.zeros_like(exact)
    for h in range(w.n_kv_heads):
        bound[:, h] = absK[:, :, h, :] @ np.abs(P[h].astype(np.float64))
    bound *= 1.01 * w.d_k * 2.0 ** -24
    g64 = O.to_f64(got)
    ex = np.clip(exact, -448.0, 448.0)
    half = _e4m3_half_step(np.maximum(np.abs(g64), np.abs(ex)))
    assert (np.abs(g64 - ex) <= bound + half).all()
    # a code other than the oracle's needs the exact value next to a midpoint
    diff = got != stored
    if diff.any():
        lo, hi = O.to_f64(np.minimum(got, stored)[diff]), O.to_f64(np.maximum(got, stored)[diff])
        mid = exact[diff]
        assert (np.abs(np.abs(mid) - (np.abs(lo) + np.abs(hi)) / 2) <= bound[diff] + 1e-30).all()


@pytest.mark.parametrize("name", ["llama", "g1r64"])
def test_fp8_projection_of_cached_rows(name):
    w = CASES[name]
    inp = inputs(w)
    desc = fdesc(w)
    kp = _kp_empty(w)
    J.append_projection(desc, w.t_max, torch.zeros(w.batch, dtype=torch.int32, device="cuda"),
                        to_dev(inp["P"]), to_dev(inp["k_cache"]), kp)
    got = to_host(kp)
    stored, exact = O.project_keys(inp["k_cache"], inp["P"], np.full(w.batch, w.t_max), "fp8")
    _check_projection_fp8(got, stored, exact, inp["k_cache"], inp["P"], w)
    assert (got != stored).mean() < 1e-3


def test_fp8_append_new_rows_and_saturation():
    """Three new rows per sequence (the few-rows kernel) and one step's row
    (the one-round-trip kernel): K/V copied, keys projected to E4M3; rows
    scaled far past 448 saturate to +-448 (codes 0x7E / 0xFE)."""
    w = CASES["llama"]
    inp = inputs(w)
    desc = fdesc(w)
    rng = np.random.default_rng(5)
    for n_new, scale in ((3, 1.0), (1, 1.0), (1, 2000.0)):
        k = to_dev(inp["k_cache"])
        v = to_dev(inp["v_cache"])
        kp = _kp_empty(w)
        pos_h = np.array([w.t_max - 5 - 7 * b for b in range(w.batch)], np.int32)
        kn = to_bf16_bits(rng.standard_normal((w.batch, n_new, w.n_kv_heads, w.d_k)).astype(np.float32) * scale)
        vn = to_bf16_bits(rng.standard_normal((w.batch, n_new, w.n_kv_heads, w.d_v)).astype(np.float32))
        J.append_kv(desc, to_dev(kn), to_dev(vn), to_dev(pos_h), to_dev(inp["P"]), k, v, kp)
        kc, vc, kpc = to_host(k), to_host(v), to_host(kp)
        ref_k, ref_v = inp["k_cache"].copy(), inp["v_cache"].copy()
        for b in range(w.batch):
            ref_k[b, pos_h[b]:pos_h[b] + n_new] = kn[b]
            ref_v[b, pos_h[b]:pos_h[b] + n_new] = vn[b]
        assert np.array_equal(kc, ref_k) and np.array_equal(vc, ref_v)
        stored, exact = O.project_keys(ref_k, inp["P"], np.full(w.batch, w.t_max), "fp8")
        for b in range(w.batch):
            rows = slice(pos_h[b], pos_h[b] + n_new)
            _check_projection_fp8(kpc[b:b + 1, :, rows], stored[b:b + 1, :, rows], exact[b:b + 1, :, rows],
                                  ref_k[b:b + 1, rows], inp["P"], w)
            mask = np.ones(w.t_max, bool)
            mask[rows] = False
            assert (kpc[b][:, mask] == 0).all()
        if scale > 1.0:
            sat = np.abs(exact) > 480.0
            assert sat.sum() > 100
            new = np.zeros_like(sat)
            for b in range(w.batch):
                new[b, :, pos_h[b]:pos_h[b] + n_new] = True
            assert (kpc[sat & new] == np.where(exact[sat & new] > 0, 0x7E, 0xFE)).all()


@pytest.mark.parametrize("reduce", [J.REDUCE_MAX, J.REDUCE_MEAN], ids=["max", "mean"])
@pytest.mark.parametrize("name", list(CASES))
def test_fp8_scores_match_oracle(name, reduce):
    w = CASES[name]
    inp = inputs(w)
    desc = fdesc(w, reduce=reduce)
    kp = oracle_kp(inp, desc)
    assert kp.dtype == np.uint8
    scores = torch.full((w.batch, w.n_kv_heads, w.t_max), 12345.0, device="cuda")
    J.score(desc, to_dev(inp["q"]), to_dev(inp["P"]), to_dev(kp), to_dev(inp["seq_lens"]), scores)
    got = to_host(scores).astype(np.float64)
    s64, n_cand = O.subspace_scores(inp["q"], inp["P"], kp, inp["seq_lens"], w.window,
                                    "max" if reduce == J.REDUCE_MAX else "mean")
    q64, P64 = np.abs(O.to_f64(inp["q"])), np.abs(inp["P"].astype(np.float64))
    G = w.group
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            n = int(n_cand[b])
            aqp = q64[b, h * G:(h + 1) * G] @ P64[h]
            bound = (np.abs(O.to_f64(kp[b, h, :n])) @ aqp.T).max(axis=1) * (w.d_k + w.rank) * 2.0 ** -23
            err = np.abs(got[b, h, :n] - s64[b, h, :n])
            assert (err <= bound + 1e-30).all(), (b, h, err.max())
            assert (got[b, h, n:] == 12345.0).all()


def _decode(desc, w, inp, kp, profiled=False):
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


def _composed(desc, w, inp, kp):
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
    return to_host(out), to_host(lse), to_host(idx), to_host(n_sel), to_host(scores)


@pytest.mark.parametrize("reduce", [J.REDUCE_MAX, J.REDUCE_MEAN], ids=["max", "mean"])
@pytest.mark.parametrize("name", list(CASES))
def test_fp8_decode_matches_oracle_and_composed(name, reduce):
    w = CASES[name]
    inp = inputs(w)
    desc = fdesc(w, reduce=reduce)
    kp = oracle_kp(inp, desc)
    o1, l1, i1, n1, _ = _decode(desc, w, inp, kp)
    o2, l2, i2, n2, _ = _composed(desc, w, inp, kp)
    assert np.array_equal(n1, n2) and np.array_equal(i1, i2)
    assert rel_l2(o1, o2) <= 1e-5
    o3, _, i3, n3, _ = _decode(desc, w, inp, kp, profiled=True)
    assert np.array_equal(i3, i1) and np.array_equal(n3, n1) and np.array_equal(o3, o1)
    s64, n_cand = O.subspace_scores(inp["q"], inp["P"], kp, inp["seq_lens"], w.window,
                                    "max" if reduce == J.REDUCE_MAX else "mean")
    check_sets_within_tolerance(i1, n1, s64, n_cand, inp["seq_lens"], w.topk, w.window)
    ref, ref_lse = O.attention(inp["q"], inp["k_cache"], inp["v_cache"], np.where(i1 < 0, 0, i1), n1, w.scale)
    assert rel_l2(o1, ref) <= 2e-3
    assert np.abs(l1 - ref_lse).max() <= 1e-4 * max(1.0, np.abs(ref_lse).max())


@pytest.mark.parametrize("n_groups", [5, 60])
def test_fp8_decode_heavy_ties(n_groups):
    """Projected keys drawn from a few distinct rows: large groups of equal
    scores around the k-th; the decode equals the composed entry points and
    the oracle's full-sort top-k on the GPU's own fp32 scores."""
    w = CASES["llama"]
    inp = inputs(w)
    desc = fdesc(w)
    kp = oracle_kp(inp, desc).copy()
    B, Hkv, T, _ = kp.shape
    rng = np.random.default_rng(13 + n_groups)
    for b in range(B):
        for h in range(Hkv):
            rows = kp[b, h, rng.choice(T, n_groups, replace=False)].copy()
            kp[b, h] = rows[rng.integers(0, n_groups, T)]
    o1, _, i1, n1, _ = _decode(desc, w, inp, kp)
    o2, _, i2, n2, s32 = _composed(desc, w, inp, kp)
    assert np.array_equal(n1, n2) and np.array_equal(i1, i2)
    ref_idx, ref_n = O.topk_select(s32.astype(np.float64), inp["seq_lens"], w.topk, w.window)
    assert np.array_equal(ref_n, n1)
    for b in range(B):
        for h in range(Hkv):
            n = int(ref_n[b, h])
            assert np.array_equal(np.sort(ref_idx[b, h, :n]), i1[b, h, :n]), (b, h)


def test_fp8_sample_threshold_fallback_is_exact():
    """The largest scores planted on the grid the threshold sample reads
    (every (n_cand // 1024)-th token: the sample is one 1024-token tile): the
    threshold admits fewer than k tokens and the row is re-selected exactly."""
    w = CASES["llama"]
    inp = inputs(w)
    desc = fdesc(w)
    kp = oracle_kp(inp, desc).copy()
    qp = O.project_query(inp["q"], inp["P"], w.n_kv_heads)
    G = w.group
    rng = np.random.default_rng(9)
    for b in range(w.batch):
        n_cand = int(inp["seq_lens"][b]) - w.window
        assert n_cand > 8192
        for h in range(w.n_kv_heads):
            v = qp[b, h * G]
            grid = np.arange(0, n_cand, n_cand // 1024)
            rows = (6.0 / np.linalg.norm(v)) * v[None, :] * (1.0 + 0.05 * rng.random((grid.size, 1)))
            kp[b, h, grid] = O.round_to_e4m3_bits(rows)
    o1, _, i1, n1, ws = _decode(desc, w, inp, kp)
    assert int(J.workspace_status(ws, clear=False).cpu()[J.STATUS_EXACT_REDO]) >= 1  # rows re-selected
    _, _, i2, n2, _ = _composed(desc, w, inp, kp)
    assert np.array_equal(i1, i2) and np.array_equal(n1, n2)
    s64, n_cand = O.subspace_scores(inp["q"], inp["P"], kp, inp["seq_lens"], w.window)
    check_sets_within_tolerance(i1, n1, s64, n_cand, inp["seq_lens"], w.topk, w.window)


@pytest.mark.parametrize("name", ["128k", "g1r64", "g2"])
def test_fp8_decode_step_equals_append_then_decode(name):
    """The one-call step with FP8 keys: the caches, indices and outputs of
    jssa_append_kv + jssa_decode, bit for bit, with the new token early, late
    and at T_b - 1 over the batch."""
    w = CASES[name]
    inp = inputs(w)
    desc = fdesc(w)
    L = inp["seq_lens"].astype(np.int64)
    n_cand = L - w.window
    pos = np.array([[n_cand[b] // 7, n_cand[b] - 4, L[b] - 1][b % 3] for b in range(w.batch)], np.int32)
    rng = np.random.default_rng(21)
    kn = to_bf16_bits(rng.standard_normal((w.batch, 1, w.n_kv_heads, w.d_k)).astype(np.float32) * 3)
    vn = to_bf16_bits(rng.standard_normal((w.batch, 1, w.n_kv_heads, w.d_v)).astype(np.float32))
    q, P, seq = to_dev(inp["q"]), to_dev(inp["P"]), to_dev(inp["seq_lens"])
    res = []
    for fused in (False, True):
        K, V, kp = to_dev(inp["k_cache"]), to_dev(inp["v_cache"]), _kp_empty(w)
        J.append_projection(desc, w.t_max, torch.zeros(w.batch, dtype=torch.int32, device="cuda"), P, K, kp)
        out = torch.empty((w.batch, w.n_q_heads, w.d_v), device="cuda")
        lse = torch.empty((w.batch, w.n_q_heads), device="cuda")
        idx = torch.full((w.batch, w.n_kv_heads, w.topk + w.window), -1, dtype=torch.int32, device="cuda")
        n_sel = torch.zeros((w.batch, w.n_kv_heads), dtype=torch.int32, device="cuda")
        ws = J.workspace(desc, J.OP_DECODE)
        if fused:
            J.decode_step(desc, to_dev(kn), to_dev(vn), to_dev(pos), q, P, kp, K, V, seq, out, lse, ws,
                          idx_out=idx, n_sel_out=n_sel)
        else:
            J.append_kv(desc, to_dev(kn), to_dev(vn), to_dev(pos), P, K, V, kp)
            J.decode(desc, q, P, kp, K, V, seq, out, lse, ws, idx_out=idx, n_sel_out=n_sel)
        torch.cuda.synchronize()
        res.append([to_host(t) for t in (kp, K, V, out, lse, n_sel)] + [to_host(idx)])
    for a, b in zip(res[0][:-1], res[1][:-1]):
        assert np.array_equal(a, b)
    gn = res[0][5]
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            assert np.array_equal(res[0][6][b, h, :gn[b, h]], res[1][6][b, h, :gn[b, h]])
