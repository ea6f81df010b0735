"""Pins of the CPU oracle to things other than itself.

Every oracle function is checked here against a closed form, exact rational
arithmetic, brute-force enumeration, a library routine or hand-derived golden
values, so that a dropped term, a wrong sign or index, or a transposed
operand in the oracle fails at least one test.  CPU only.
"""
import itertools
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.special
import scipy.stats
import torch

from oracle import jssa_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bf16_bits_torch(x32: np.ndarray) -> np.ndarray:
    return torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _small_int_bf16(rng, shape, lo=-8, hi=9):
    """Small integers: exact in bf16, fp32 and fp64, so sums are exact too."""
    v = rng.integers(lo, hi, size=shape).astype(np.float32)
    return _bf16_bits_torch(v), v.astype(np.int64)


# ----------------------------------------------------------------------------- bf16 rounding
def test_bf16_rounding_golden():
    """Hand-derived round-to-nearest-even cases, including ones where rounding
    through float32 first (double rounding) would give a different answer."""
    rows = []
    with open(os.path.join(GOLDEN, "bf16_rne.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            val, bits = line.split()[:2]
            rows.append((float.fromhex(val), int(bits, 16)))
    x = np.array([r[0] for r in rows])
    want = np.array([r[1] for r in rows], np.uint16)
    got = O.round_to_bf16_bits(x)
    assert (got == want).all(), list(zip(x, got, want))
    assert len(rows) >= 15


def test_bf16_rounding_matches_library_on_float32_values():
    """For float32 inputs a single rounding equals torch's float32->bfloat16 conversion."""
    rng = np.random.default_rng(7)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(3.0),
        rng.integers(0, 2**32, 20000, dtype=np.uint64).astype(np.uint32).view(np.float32),
        np.array([0.0, -0.0, np.inf, -np.inf, 1e-40, -1e-42, 3.4e38, -3.39e38], np.float32),
    ])
    x = x[np.isfinite(x) | np.isinf(x)]  # drop NaN payloads (checked separately)
    got = O.round_to_bf16_bits(x.astype(np.float64))
    want = _bf16_bits_torch(x)
    assert (got == want).all()
    assert O.round_to_bf16_bits(np.array([np.nan]))[0] & 0x7F80 == 0x7F80


def test_to_f64_decodes_bits():
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x0001, 0x7F80, 0xFF80], np.uint16)
    want = [1.0, -1.0, 3.140625, 2.0 ** -133, np.inf, -np.inf]
    assert O.to_f64(bits).tolist() == want


# ----------------------------------------------------------------------------- FP8 E4M3
def test_e4m3_rounding_golden():
    """Hand-derived E4M3 round-to-nearest-even cases: ties, subnormals, the
    largest value and saturation."""
    rows = []
    with open(os.path.join(GOLDEN, "e4m3_rne.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            val, code = line.split()[:2]
            rows.append((float.fromhex(val), int(code, 16)))
    x = np.array([r[0] for r in rows])
    want = np.array([r[1] for r in rows], np.uint8)
    got = O.round_to_e4m3_bits(x)
    assert (got == want).all(), list(zip(x, got, want))
    assert len(rows) >= 20


def test_e4m3_decoding_matches_format_definition_and_library():
    """All 256 codes: the OFP8 E4M3 definition written out with exact
    rationals, and torch's float8_e4m3fn reading of the same bytes."""
    codes = np.arange(256, dtype=np.uint8)
    got = O.e4m3_to_f64(codes)
    for c in range(256):
        s, e, m = c >> 7, (c >> 3) & 15, c & 7
        if e == 15 and m == 7:
            assert math.isnan(got[c])
            continue
        mag = Fraction(m, 8) * Fraction(2) ** -6 if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
        assert got[c] == float(-mag if s else mag) and math.copysign(1.0, got[c]) == (-1.0 if s else 1.0)
    lib = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    assert np.array_equal(np.isnan(got), np.isnan(lib))
    assert np.array_equal(got[~np.isnan(got)], lib[~np.isnan(lib)])
    assert np.nanmax(got) == 448.0 and np.nanmin(got) == -448.0
    assert O.to_f64(np.array([0x38, 0xC0], np.uint8)).tolist() == [1.0, -2.0]


def test_e4m3_rounding_brute_force_and_library():
    """Every code rounds back to itself; every midpoint between neighbouring
    values goes to the even code and points just beside it to the nearer one;
    inside the range the rounding equals torch's float32 -> float8_e4m3fn
    conversion; beyond it, it saturates."""
    codes = np.arange(256, dtype=np.uint8)
    vals = O.e4m3_to_f64(codes)
    finite = ~np.isnan(vals)
    assert (O.round_to_e4m3_bits(vals[finite]) == codes[finite]).all()
    pos = np.unique(vals[finite & (vals >= 0)])
    for a, b in zip(pos[:-1], pos[1:]):
        ca, cb = O.round_to_e4m3_bits(np.array([a, b]))
        mid = (a + b) / 2
        even = ca if ca % 2 == 0 else cb
        assert O.round_to_e4m3_bits(np.array([mid]))[0] == even
        assert O.round_to_e4m3_bits(np.array([-mid]))[0] == even | 0x80
        eps = (b - a) * 2.0 ** -20
        assert O.round_to_e4m3_bits(np.array([mid - eps, mid + eps])).tolist() == [ca, cb]
    rng = np.random.default_rng(11)
    x = np.concatenate([rng.standard_normal(50000) * 3.0, rng.standard_normal(20000) * 0.01,
                        rng.uniform(-448.0, 448.0, 20000)]).astype(np.float32)
    lib = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert (O.round_to_e4m3_bits(x.astype(np.float64)) == lib).all()
    big = np.array([464.0, 470.0, 1e6, np.inf, -500.0, -np.inf])
    assert O.round_to_e4m3_bits(big).tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE]
    assert O.round_to_e4m3_bits(np.array([np.nan]))[0] == 0x7F
    assert O.round_to_e4m3_bits(np.array([0.0, -0.0])).tolist() == [0x00, 0x80]


# ----------------------------------------------------------------------------- key projection
def test_project_keys_identity_basis_is_exact():
    """r = d and P = I: the projected cache holds the keys bit for bit."""
    rng = np.random.default_rng(1)
    B, T, Hkv, d = 2, 37, 3, 16
    K = _bf16_bits_torch(rng.standard_normal((B, T, Hkv, d)).astype(np.float32))
    P = np.broadcast_to(np.eye(d, dtype=np.float32), (Hkv, d, d)).copy()
    seq = np.array([37, 20], np.int32)
    kp, exact = O.project_keys(K, P, seq, "bf16")
    for b in range(B):
        n = seq[b]
        assert (kp[b, :, :n, :] == K[b, :n].transpose(1, 0, 2)).all()
        assert (kp[b, :, n:, :] == 0).all()


def test_project_keys_exact_rational():
    """Kp = K P per KV head, checked with exact rational sums of the float values."""
    rng = np.random.default_rng(2)
    B, T, Hkv, d, r = 1, 5, 2, 8, 3
    K = rng.standard_normal((B, T, Hkv, d)).astype(np.float32)
    P = np.stack([scipy.stats.ortho_group.rvs(d, random_state=10 + h)[:, :r] for h in range(Hkv)]).astype(np.float32)
    _, exact = O.project_keys(K, P, np.array([T], np.int32), "f32")
    for h in range(Hkv):
        for t in range(T):
            for i in range(r):
                ref = sum(Fraction(float(K[0, t, h, j])) * Fraction(float(P[h, j, i])) for j in range(d))
                assert abs(exact[0, h, t, i] - float(ref)) <= 1e-12 * (1 + abs(float(ref)))


def test_project_keys_bf16_is_single_rounding_of_exact_product():
    rng = np.random.default_rng(3)
    K = rng.standard_normal((1, 64, 2, 32)).astype(np.float32)
    P = np.stack([scipy.stats.ortho_group.rvs(32, random_state=h)[:, :8] for h in range(2)]).astype(np.float32)
    kp, exact = O.project_keys(K, P, np.array([64], np.int32), "bf16")
    v = O.to_f64(kp)
    # nearest: no bf16 value lies strictly closer to the exact product
    up = O.to_f64(kp + np.uint16(1))
    dn = O.to_f64(kp - np.uint16(1))
    assert (np.abs(v - exact) <= np.abs(up - exact)).all()
    assert (np.abs(v - exact) <= np.abs(dn - exact)).all()


def test_project_keys_fp8_is_single_rounding_of_exact_product():
    """FP8 store: the nearest E4M3 value to the exact product (no code lies
    strictly closer), saturating; the identity basis reproduces keys that are
    E4M3 values."""
    rng = np.random.default_rng(4)
    K = (rng.standard_normal((1, 64, 2, 32)) * 4.0).astype(np.float32)
    P = np.stack([scipy.stats.ortho_group.rvs(32, random_state=20 + h)[:, :8] for h in range(2)]).astype(np.float32)
    kp, exact = O.project_keys(K, P, np.array([64], np.int32), "fp8")
    assert kp.dtype == np.uint8
    v = O.to_f64(kp)
    allv = O.e4m3_to_f64(np.arange(256, dtype=np.uint8))
    allv = allv[~np.isnan(allv)]
    nearest = np.abs(exact[..., None] - allv).min(axis=-1)
    assert (np.abs(v - exact) == nearest).all()
    # identity basis on keys that are E4M3 values: stored bit for bit
    codes = rng.integers(0, 256, size=(1, 9, 2, 8)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x38
    Kv = O.e4m3_to_f64(codes).astype(np.float32)
    Pi = np.broadcast_to(np.eye(8, dtype=np.float32), (2, 8, 8)).copy()
    kpi, _ = O.project_keys(Kv, Pi, np.array([9], np.int32), "fp8")
    want = codes[0].transpose(1, 0, 2)
    want = np.where(want == 0x80, 0x00, want)  # -0.0 * 1 + 0.0 * ... sums to +0.0
    assert (kpi[0] == want).all()


# ----------------------------------------------------------------------------- scores
def _channel_selection_basis(d, r, channels_per_head):
    """Selecting r original channels is a restricted orthonormal projection
    (JSSA summary section 2.1)."""
    Hkv = len(channels_per_head)
    P = np.zeros((Hkv, d, r), np.float32)
    for h, ch in enumerate(channels_per_head):
        for i, c in enumerate(ch):
            P[h, c, i] = 1.0
    return P


@pytest.mark.parametrize("reduce", ["max", "mean"])
def test_scores_channel_selection_closed_form(reduce):
    """With P selecting channels C_h, the subspace score is max (or mean) over the
    group's heads of sum_{c in C_h} q[c] K[c], computed here in exact integers."""
    rng = np.random.default_rng(4)
    B, T, Hkv, G, d, r = 2, 19, 2, 3, 8, 3
    chans = [[5, 0, 6], [1, 7, 2]]
    P = _channel_selection_basis(d, r, chans)
    Kb, Ki = _small_int_bf16(rng, (B, T, Hkv, d))
    qb, qi = _small_int_bf16(rng, (B, Hkv * G, d))
    seq = np.array([19, 11], np.int32)
    kp, _ = O.project_keys(Kb, P, seq, "bf16")
    s, n_cand = O.subspace_scores(qb, P, kp, seq, 0, reduce)
    assert n_cand.tolist() == [19, 11]
    for b in range(B):
        for h in range(Hkv):
            for t in range(T):
                if t >= seq[b]:
                    assert np.isnan(s[b, h, t])
                    continue
                per = [sum(int(qi[b, h * G + g, c]) * int(Ki[b, t, h, c]) for c in chans[h]) for g in range(G)]
                want = max(per) if reduce == "max" else Fraction(sum(per), G)
                assert s[b, h, t] == float(want)


def test_scores_full_rank_identity_equals_exact_dot():
    """r = d, P = I: the subspace score is the exact max over the group of q.k."""
    rng = np.random.default_rng(5)
    B, T, Hkv, G, d = 1, 23, 2, 4, 16
    P = np.broadcast_to(np.eye(d, dtype=np.float32), (Hkv, d, d)).copy()
    Kb, Ki = _small_int_bf16(rng, (B, T, Hkv, d))
    qb, qi = _small_int_bf16(rng, (B, Hkv * G, d))
    seq = np.array([T], np.int32)
    kp, _ = O.project_keys(Kb, P, seq, "bf16")
    s, _ = O.subspace_scores(qb, P, kp, seq, 0, "max")
    for h in range(Hkv):
        for t in range(T):
            want = max(int(np.dot(qi[0, h * G + g], Ki[0, t, h])) for g in range(G))
            assert s[0, h, t] == want


def test_scores_invariant_under_rotation_of_basis():
    """Replacing P by P R (R orthogonal r x r) spans the same subspace: scores unchanged."""
    rng = np.random.default_rng(6)
    B, T, Hkv, G, d, r = 1, 50, 2, 2, 16, 5
    K = rng.standard_normal((B, T, Hkv, d))
    q = rng.standard_normal((B, Hkv * G, d))
    P = np.stack([scipy.stats.ortho_group.rvs(d, random_state=h)[:, :r] for h in range(Hkv)])
    R = np.stack([scipy.stats.ortho_group.rvs(r, random_state=50 + h) for h in range(Hkv)])
    PR = np.einsum("hdr,hrs->hds", P, R)
    seq = np.array([T], np.int32)
    for reduce in ("max", "mean"):
        _, e1 = O.project_keys(K, P, seq, "f32")
        _, e2 = O.project_keys(K, PR, seq, "f32")
        s1, _ = O.subspace_scores(q, P, e1, seq, 0, reduce)
        s2, _ = O.subspace_scores(q, PR, e2, seq, 0, reduce)
        assert np.allclose(s1, s2, rtol=1e-11, atol=1e-11)
        # and a different subspace does change them
        P3 = np.stack([scipy.stats.ortho_group.rvs(d, random_state=90 + h)[:, :r] for h in range(Hkv)])
        _, e3 = O.project_keys(K, P3, seq, "f32")
        s3, _ = O.subspace_scores(q, P3, e3, seq, 0, reduce)
        assert not np.allclose(s1, s3, rtol=1e-3)


def test_scores_mean_vs_max_relations():
    rng = np.random.default_rng(8)
    B, T, Hkv, G, d, r = 2, 40, 2, 4, 16, 4
    K = rng.standard_normal((B, T, Hkv, d)).astype(np.float32)
    P = np.stack([scipy.stats.ortho_group.rvs(d, random_state=h)[:, :r] for h in range(Hkv)]).astype(np.float32)
    q = rng.standard_normal((B, Hkv * G, d)).astype(np.float32)
    seq = np.array([T, T], np.int32)
    kp, _ = O.project_keys(K, P, seq, "f32")
    smax, _ = O.subspace_scores(q, P, kp, seq, 0, "max")
    smean, _ = O.subspace_scores(q, P, kp, seq, 0, "mean")
    assert (smax >= smean - 1e-12).all() and (smax > smean + 1e-6).any()
    # identical query heads within each group: max == mean
    q_same = np.repeat(q[:, ::G], G, axis=1)
    a, _ = O.subspace_scores(q_same, P, kp, seq, 0, "max")
    m, _ = O.subspace_scores(q_same, P, kp, seq, 0, "mean")
    assert np.allclose(a, m, rtol=1e-13, atol=1e-13)


def test_scores_respect_lengths_and_window():
    rng = np.random.default_rng(9)
    B, T, Hkv, G, d, r = 3, 30, 1, 2, 8, 2
    K = rng.standard_normal((B, T, Hkv, d)).astype(np.float32)
    P = np.stack([np.eye(d, dtype=np.float32)[:, :r]])
    q = rng.standard_normal((B, Hkv * G, d)).astype(np.float32)
    seq = np.array([30, 7, 3], np.int32)
    kp, _ = O.project_keys(K, P, seq, "f32")
    s, n_cand = O.subspace_scores(q, P, kp, seq, 4, "max")
    assert n_cand.tolist() == [26, 3, 0]
    for b in range(B):
        assert np.isfinite(s[b, 0, :n_cand[b]]).all()
        assert np.isnan(s[b, 0, n_cand[b]:]).all()


# ----------------------------------------------------------------------------- selection
def _better(si, i, sj, j):
    """Strict ranking used by the selection rule: larger score, ties to the lower index,
    NaN below every number."""
    ni, nj = math.isnan(si), math.isnan(sj)
    if ni and nj:
        return i < j
    if ni != nj:
        return nj
    if si != sj:
        return si > sj
    return i < j


def _brute_force_topk(s, k):
    n = len(s)
    kk = min(k, n)
    winners = []
    for S in itertools.combinations(range(n), kk):
        rest = [j for j in range(n) if j not in S]
        if all(_better(s[i], i, s[j], j) for i in S for j in rest):
            winners.append(list(S))
    assert len(winners) == 1, winners  # the rule admits exactly one set
    return winners[0]


def test_topk_matches_brute_force_enumeration():
    rng = np.random.default_rng(10)
    specials = np.array([0.0, -0.0, np.inf, -np.inf, np.nan])
    for trial in range(300):
        T = int(rng.integers(1, 13))
        k = int(rng.integers(1, T + 2))
        W = int(rng.integers(0, 3)) if trial % 3 == 0 else 0
        s = rng.integers(-3, 4, size=T).astype(np.float64)  # many exact ties
        mask = rng.random(T) < 0.2
        s[mask] = rng.choice(specials, size=mask.sum())
        if W >= T:
            W = 0
        arr = s[None, None, :]
        idx, n_sel = O.topk_select(arr, np.array([T]), k, W)
        want = _brute_force_topk(list(s[:T - W]), k) + list(range(T - W, T))
        assert n_sel[0, 0] == len(want) == O.n_selected(T, k, W)
        assert idx[0, 0, :n_sel[0, 0]].tolist() == want
        assert (idx[0, 0, n_sel[0, 0]:] == -1).all()


def test_topk_golden_cases():
    with open(os.path.join(GOLDEN, "topk_ties.txt")) as f:
        lines = [ln for ln in f if ln.strip() and not ln.startswith("#")]
    assert len(lines) >= 10
    for ln in lines:
        k, W, scores, want = [p.strip() for p in ln.split("|")]
        s = np.array([float(x) for x in scores.split(",")])
        idx, n_sel = O.topk_select(s[None, None, :], np.array([s.size]), int(k), int(W))
        got = idx[0, 0, :n_sel[0, 0]].tolist()
        assert got == [int(x) for x in want.split(",")], ln


def test_topk_all_equal_takes_lowest_indices():
    s = np.full((2, 3, 1000), 0.5)
    idx, n_sel = O.topk_select(s, np.array([1000, 600]), 64, 0)
    assert (n_sel == 64).all()
    assert (idx == np.arange(64)).all()


def test_topk_budget_covers_all_candidates():
    rng = np.random.default_rng(11)
    s = rng.standard_normal((1, 2, 50))
    idx, n_sel = O.topk_select(s, np.array([40]), 100, 5)
    assert (n_sel == 40).all()
    assert (idx[0, :, :40] == np.arange(40)).all()


# ----------------------------------------------------------------------------- attention
def _sdpa_reference(q, K, V, scale):
    """torch's fp64 scaled_dot_product_attention on the CPU (a library routine)."""
    qt = torch.from_numpy(q)[:, :, None, :]  # [B, Hq, 1, d]
    G = q.shape[1] // K.shape[2]
    kt = torch.from_numpy(K).permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
    vt = torch.from_numpy(V).permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)
    return o[:, :, 0, :].numpy()


def test_dense_attention_matches_library_sdpa():
    rng = np.random.default_rng(12)
    B, T, Hkv, G, d, dv = 2, 77, 2, 4, 32, 24
    q = rng.standard_normal((B, Hkv * G, d))
    K = rng.standard_normal((B, T, Hkv, d))
    V = rng.standard_normal((B, T, Hkv, dv))
    out, lse = O.dense_attention(q, K, V, np.array([T, T]), 0.3)
    ref = _sdpa_reference(q, K, V, 0.3)
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-12)
    # lse against scipy's logsumexp
    for b in range(B):
        for hq in range(Hkv * G):
            logits = 0.3 * (K[b, :, hq // G, :] @ q[b, hq])
            assert abs(lse[b, hq] - scipy.special.logsumexp(logits)) < 1e-12


def test_dense_attention_ragged_lengths():
    rng = np.random.default_rng(13)
    B, T, Hkv, G, d = 2, 40, 1, 2, 8
    q = rng.standard_normal((B, Hkv * G, d))
    K = rng.standard_normal((B, T, Hkv, d))
    V = rng.standard_normal((B, T, Hkv, d))
    out, _ = O.dense_attention(q, K, V, np.array([40, 13]), 0.5)
    ref = _sdpa_reference(q[1:], K[1:, :13], V[1:, :13], 0.5)
    assert np.allclose(out[1], ref[0], rtol=1e-12, atol=1e-12)


def test_sparse_attention_with_full_budget_is_dense():
    """k = T (no window): every token is selected and sparse decode equals dense."""
    rng = np.random.default_rng(14)
    B, T, Hkv, G, d, r = 2, 64, 2, 4, 16, 4
    q = rng.standard_normal((B, Hkv * G, d)).astype(np.float32)
    K = rng.standard_normal((B, T, Hkv, d)).astype(np.float32)
    V = rng.standard_normal((B, T, Hkv, d)).astype(np.float32)
    P = np.stack([scipy.stats.ortho_group.rvs(d, random_state=h)[:, :r] for h in range(Hkv)]).astype(np.float32)
    seq = np.array([T, 50], np.int32)
    kp, _ = O.project_keys(K, P, seq, "f32")
    res = O.decode(q, P, kp, K, V, seq, T, 0, 0.25)
    ref = _sdpa_reference(q.astype(np.float64)[:1], K[:1].astype(np.float64), V[:1].astype(np.float64), 0.25)
    assert np.allclose(res["out"][0], ref[0], rtol=1e-12, atol=1e-12)
    ref1 = _sdpa_reference(q.astype(np.float64)[1:], K[1:, :50].astype(np.float64), V[1:, :50].astype(np.float64), 0.25)
    assert np.allclose(res["out"][1], ref1[0], rtol=1e-12, atol=1e-12)


def test_single_selected_token_returns_its_value_row():
    rng = np.random.default_rng(15)
    q = rng.standard_normal((1, 4, 8))
    K = rng.standard_normal((1, 10, 2, 8))
    V = rng.standard_normal((1, 10, 2, 6))
    idx = np.array([[[7], [2]]], np.int32)
    out, lse = O.attention(q, K, V, idx, np.ones((1, 2), np.int32), 0.7)
    for hq in range(4):
        h = hq // 2
        t = idx[0, h, 0]
        assert (out[0, hq] == V[0, t, h]).all()
        assert abs(lse[0, hq] - 0.7 * float(np.dot(K[0, t, h], q[0, hq]))) < 1e-13


def test_attention_uses_selected_rows_only_and_is_order_free():
    rng = np.random.default_rng(16)
    B, T, Hkv, G, d = 1, 30, 2, 2, 8
    q = rng.standard_normal((B, Hkv * G, d))
    K = rng.standard_normal((B, T, Hkv, d))
    V = rng.standard_normal((B, T, Hkv, d))
    idx = np.array([[[3, 9, 20, 21], [0, 5, 6, 29]]], np.int32)
    n = np.full((1, 2), 4, np.int32)
    out, _ = O.attention(q, K, V, idx, n, 0.4)
    out2, _ = O.attention(q, K, V, idx[:, :, ::-1].copy(), n, 0.4)
    assert np.allclose(out, out2, rtol=1e-13, atol=1e-13)
    for h in range(Hkv):
        rows = idx[0, h]
        ref = _sdpa_reference(q[:, h * G:(h + 1) * G], K[:, rows][:, :, h:h + 1], V[:, rows][:, :, h:h + 1], 0.4)
        assert np.allclose(out[0, h * G:(h + 1) * G], ref[0], rtol=1e-12, atol=1e-12)


def test_mla_shared_latent_row_values():
    """MLA (JSSA summary section 3.3): one latent row per token; the value is its
    first d_v columns.  Checked against SDPA with v = k[..., :d_v]."""
    rng = np.random.default_rng(17)
    B, T, Hq, dk, dv = 1, 40, 16, 24, 16
    q = rng.standard_normal((B, Hq, dk))
    L = rng.standard_normal((B, T, 1, dk))
    out, _ = O.dense_attention(q, L, L[..., :dv], np.array([T]), 0.2)
    ref = _sdpa_reference(q, L, np.ascontiguousarray(L[..., :dv]), 0.2)
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-12)


def test_gather_then_dense_attention_equals_indexed_attention():
    """Dense attention over the packed rows equals the indexed attention over
    the same lists (ragged counts, repeated and unsorted indices, MLA's one
    list per sequence), and the packed rows are the indexed rows."""
    rng = np.random.default_rng(17)
    B, T, Hkv, G, d = 3, 40, 2, 3, 8
    K = rng.standard_normal((B, T, Hkv, d)).astype(np.float32)
    V = rng.standard_normal((B, T, Hkv, d)).astype(np.float32)
    q = rng.standard_normal((B, Hkv * G, d)).astype(np.float32)
    S = 12
    idx = rng.integers(0, T, size=(B, Hkv, S)).astype(np.int32)
    n_sel = np.array([[12, 12], [5, 5], [0, 0]], np.int32)
    Kg, Vg = O.gather_rows(K, idx, n_sel), O.gather_rows(V, idx, n_sel)
    for b in range(B):
        for h in range(Hkv):
            for i in range(S):
                want = K[b, idx[b, h, i], h] if i < n_sel[b, h] else np.zeros(d, np.float32)
                assert np.array_equal(Kg[b, i, h], want)
    ref, ref_lse = O.attention(q, K, V, idx, n_sel, 0.3)
    got, got_lse = O.dense_attention(q, Kg, Vg, n_sel[:, 0], 0.3)
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12)
    fin = np.isfinite(ref_lse)
    assert np.array_equal(fin, np.isfinite(got_lse)) and np.allclose(got_lse[fin], ref_lse[fin], rtol=1e-12)
    # MLA: one latent row per token, the value a prefix of it
    L = rng.standard_normal((B, T, 1, d)).astype(np.float32)
    qm = rng.standard_normal((B, 4, d)).astype(np.float32)
    Lg = O.gather_rows(L, idx[:, :1], n_sel[:, :1])
    ref, _ = O.attention(qm, L, L[..., :5], idx[:, :1], n_sel[:, :1], 0.5)
    got, _ = O.dense_attention(qm, Lg, Lg[..., :5], n_sel[:, 0], 0.5)
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_soft_vote_pins():
    """Head-shared soft voting against its definition's consequences: each
    head's votes sum to one (the total is Hkv); one head's vote ranks tokens
    as its scores do (so the shared set is that head's top-k); adding a
    constant to a head's scores changes nothing; a hand-computed two-head
    case; candidates only (window and padding excluded); NaN scores vote 0."""
    rng = np.random.default_rng(23)
    B, Hkv, T = 2, 3, 50
    s = rng.standard_normal((B, Hkv, T))
    seq = np.array([50, 31])
    v = O.soft_vote(s, seq, 5, 0.7)
    assert np.allclose(np.nansum(v[:, 0], axis=1), [Hkv, Hkv], rtol=1e-12)
    assert np.isnan(v[0, 0, 45:]).all() and np.isnan(v[1, 0, 26:]).all() and not np.isnan(v[1, 0, :26]).any()
    one = O.soft_vote(s[:, :1], seq, 5, 0.7)
    i1, n1 = O.topk_select(one, seq, 7, 5)
    i0, n0 = O.topk_select(s[:, :1], seq, 7, 5)
    assert np.array_equal(i1, i0) and np.array_equal(n1, n0)
    shifted = s.copy()
    shifted[:, 1] += 3.25
    assert np.allclose(O.soft_vote(shifted, seq, 5, 0.7), v, rtol=1e-12, equal_nan=True)
    # two heads, three tokens, scale 1: vote = softmax(h0) + softmax(h1)
    hand = np.array([[[0.0, np.log(3.0), 0.0], [np.log(2.0), 0.0, np.log(2.0)]]])
    got = O.soft_vote(hand, np.array([3]), 0, 1.0)[0, 0]
    assert np.allclose(got, [1 / 5 + 2 / 5, 3 / 5 + 1 / 5, 1 / 5 + 2 / 5], rtol=1e-12)
    nan = s.copy()
    nan[0, :, 3] = np.nan
    vn = O.soft_vote(nan, seq, 5, 0.7)
    assert vn[0, 0, 3] == 0.0 and np.isclose(np.nansum(vn[0, 0]), Hkv)


def _stack_layers(rng, n_layers, B, T, Hkv, G, d, r):
    layers = []
    for _ in range(n_layers):
        P = np.stack([scipy.stats.ortho_group.rvs(d, random_state=int(rng.integers(1 << 30)))[:, :r]
                      for _ in range(Hkv)]).astype(np.float32)
        layers.append({"q": rng.standard_normal((B, Hkv * G, d)).astype(np.float32),
                       "k_cache": rng.standard_normal((B, T, Hkv, d)).astype(np.float32),
                       "v_cache": rng.standard_normal((B, T, Hkv, d)).astype(np.float32), "P": P})
    return layers


def test_layer_stack_reuse_pins():
    """Layers that reuse an indexer layer's lists (JSSA summary appendix C)."""
    rng = np.random.default_rng(31)
    B, T, Hkv, G, d, r = 2, 48, 2, 2, 8, 4
    seq = np.array([48, 30], np.int32)
    topk, W, scale = 10, 4, 0.4
    layers = _stack_layers(rng, 4, B, T, Hkv, G, d, r)
    for L in layers:
        L["kp_cache"], _ = O.project_keys(L["k_cache"], L["P"], seq, "f32")
    res = O.layer_stack_decode(layers, seq, topk, W, scale, indexer_every=2)
    assert [x["indexer"] for x in res] == [True, False, True, False]
    for li in (1, 3):
        idx, n_sel = res[li - 1]["idx"], res[li - 1]["n_sel"]
        assert np.array_equal(res[li]["idx"], idx)
        # the reuse layer's own selection differs, so the pin below tells the lists apart
        own = O.decode(layers[li]["q"], layers[li]["P"], layers[li]["kp_cache"], layers[li]["k_cache"],
                       layers[li]["v_cache"], seq, topk, W, scale)
        assert not np.array_equal(own["idx"], idx)
        # softmax (scipy) over its own rows at the indexer's positions
        L = layers[li]
        for b in range(B):
            for hq in range(Hkv * G):
                h = hq // G
                sel = idx[b, h, :n_sel[b, h]]
                logits = scale * (L["k_cache"][b, sel, h].astype(np.float64) @ L["q"][b, hq].astype(np.float64))
                ref = scipy.special.softmax(logits) @ L["v_cache"][b, sel, h].astype(np.float64)
                assert np.allclose(res[li]["out"][b, hq], ref, rtol=1e-12, atol=1e-12)
                assert abs(res[li]["lse"][b, hq] - scipy.special.logsumexp(logits)) < 1e-12
    # a reuse layer with the indexer layer's own query and caches gives its result exactly
    twin = [layers[0], {k: layers[0][k] for k in ("q", "k_cache", "v_cache")}]
    r2 = O.layer_stack_decode(twin, seq, topk, W, scale, indexer_every=2)
    assert np.array_equal(r2[1]["out"], r2[0]["out"]) and np.array_equal(r2[1]["lse"], r2[0]["lse"])
    # a budget covering every token: every layer, reused or not, is dense attention (torch SDPA)
    full = O.layer_stack_decode(layers, np.array([T, T], np.int32), T, 0, scale, indexer_every=3)
    for li, L in enumerate(layers):
        ref = _sdpa_reference(L["q"].astype(np.float64), L["k_cache"].astype(np.float64),
                              L["v_cache"].astype(np.float64), scale)
        assert np.allclose(full[li]["out"], ref, rtol=1e-12, atol=1e-12)


def test_write_new_rows():
    cache = np.arange(2 * 5 * 2 * 3, dtype=np.float32).reshape(2, 5, 2, 3)
    new = -np.ones((2, 1, 2, 3), np.float32)
    out = O.write_new_rows(cache, new, np.array([3, 5]))  # sequence 1: past t_max, not written
    assert (out[0, 3] == -1).all()
    keep = np.ones(cache.shape, bool)
    keep[0, 3] = False
    assert np.array_equal(out[keep], cache[keep])
    assert np.array_equal(O.write_new_rows(cache, new, np.array([-1, 5])), cache)


def test_kth_score():
    s = np.array([5.0, 1.0, 5.0, 3.0, np.nan])
    assert O.kth_score(s, 5, 1) == 5.0
    assert O.kth_score(s, 5, 3) == 3.0
    assert O.kth_score(s, 5, 9) == 1.0 or np.isnan(O.kth_score(s, 5, 9))
