"""GPU parity at the full sizes of the two headline decode workloads, in the
launch configuration the benchmark times (one ``jssa_decode_step``): the
128K-context GQA step (batch 4, 32 query / 8 KV heads, d = 128, r = 32,
k = 2048) and the MLA step (batch 8, 128
query heads sharing one 576-wide latent row, r = 64, k = 2048). As in the
benchmark, the GPU projects the whole key cache, then appends one new token at
T_b - 1 and decodes in one call on the decode workspace (also with FP8
projected keys).

The oracle checks (sequence, KV head) rows one at a time (every row of the
128K bf16 step and of the MLA step, 32 rows of the ragged batch, 8 of each
other variant): it projects
that row's keys itself, and the row's projected keys in the GPU cache are
replaced by the oracle's before the decode, so both sides score the same
input (rows are independent in the decode). Every other row is checked by
properties that hold at any size: selection counts, strictly ascending indices
inside the sequence, finite outputs."""
import numpy as np
import pytest
import torch

import token_level_sparse_dim_amd as J
from oracle import jssa_oracle as O
from synth import WORKLOADS, generate, scaled, to_bf16_bits

from _gpu_helpers import check_sets_within_tolerance, desc_for, rel_l2, to_dev, to_host

pytestmark = pytest.mark.gpu

ATT_TOL = 2e-3  # bf16 inputs, fp32 accumulation


def _new_token(w, seed):
    """One new key (and value) row per sequence, drawn as the benchmark draws it."""
    rng = np.random.default_rng(seed)
    kn = rng.standard_normal((w.batch, 1, w.n_kv_heads, w.d_k)).astype(np.float32)
    vn = rng.standard_normal((w.batch, 1, w.n_kv_heads, w.d_v)).astype(np.float32)
    return to_bf16_bits(kn), to_bf16_bits(vn)


def _check_row_projection(got, k_rows, P_h, w, kp="bf16"):
    """GPU projection of one row = the fp32-accumulated K.P rounded to the
    cache type (bf16, or FP8 E4M3 saturating at 448): within the recursive
    summation bound plus half a step of the fp64 product, and the oracle's
    correctly rounded value except next to a rounding boundary. (The fraction
    is checked on whole rows; a single appended token only gets the bound.)
    Returns the oracle's stored row."""
    stored, exact = O.project_keys(k_rows[None, :, None, :], P_h[None], np.array([k_rows.shape[0]]), kp)
    stored, exact = stored[0, 0], exact[0, 0]
    g64 = O.to_f64(got)
    bound = np.abs(O.to_f64(k_rows)) @ np.abs(P_h.astype(np.float64)) * (1.01 * w.d_k * 2.0 ** -24)
    if kp == "fp8":
        exact = np.clip(exact, -448.0, 448.0)
        e = np.maximum(np.frexp(np.maximum(np.abs(g64), np.abs(exact)))[1] - 1, -6)
        half_step = np.ldexp(1.0, e - 4)
    else:
        half_step = np.ldexp(1.0, np.frexp(np.maximum(np.abs(g64), np.abs(exact)))[1] - 9)
    assert (np.abs(g64 - exact) <= bound + half_step).all()
    if got.shape[0] >= 1024:
        assert (got != stored).mean() < 1e-3
    return stored


def _check_structure(gi, gn, L, w):
    """Properties of every row: the selection count, strictly ascending
    indices inside the sequence, the window at the end."""
    B, Hkv = gn.shape
    for b in range(B):
        n_cand = max(int(L[b]) - w.window, 0)
        n_exp = min(w.window, int(L[b])) + min(w.topk, n_cand)
        for h in range(Hkv):
            assert int(gn[b, h]) == n_exp, (b, h, int(gn[b, h]), n_exp)
            sel = gi[b, h, :n_exp]
            assert (np.diff(sel) > 0).all() and sel[0] >= 0 and sel[-1] < L[b]
            if w.window:
                assert np.array_equal(sel[n_exp - w.window:], np.arange(L[b] - w.window, L[b]))


def _eight(w):
    """Eight rows spread over the sequences and KV heads."""
    return [(b % w.batch, (3 * b + 1) % w.n_kv_heads) for b in range(8)]


def _run_full(w, samples, reduce=J.REDUCE_MAX, kp_dtype=J.BF16, pos_of=None):
    """samples: (sequence, KV head) pairs, or a function of the sequence
    lengths that returns them; pos_of: the new token's position per sequence
    from the lengths (default T_b - 1, as the benchmark appends it).  Returns
    the decode workspace's diagnostic words."""
    inp = generate(w, seed=w.seed)  # the benchmark's first input set
    desc = desc_for(w, reduce=reduce, kp_dtype=kp_dtype)
    kps = "fp8" if kp_dtype == J.FP8_E4M3 else "bf16"
    B, Hkv, T, r, G = w.batch, w.n_kv_heads, w.t_max, w.rank, w.group
    L = inp["seq_lens"]
    if callable(samples):
        samples = samples(L)
    pos_h = (L - 1 if pos_of is None else pos_of(L)).astype(np.int32)
    assert ((pos_h >= 0) & (pos_h < L)).all()
    dev = "cuda"
    q, P, K, seq = (to_dev(inp[k]) for k in ("q", "P", "k_cache", "seq_lens"))
    V = None if w.mla else to_dev(inp["v_cache"])

    # (1) the whole-cache projection the benchmark starts from; the sampled rows
    # are checked and then replaced by the oracle's own projection
    kp = torch.empty((B, Hkv, T, r), dtype=torch.uint8 if kps == "fp8" else torch.bfloat16, device=dev)
    J.append_projection(desc, T, torch.zeros(B, dtype=torch.int32, device=dev), P, K, kp)
    torch.cuda.synchronize()
    kp_ref = {}
    for b, h in samples:
        n = int(L[b])
        got = to_host(kp[b, h, :n])
        kp_ref[b, h] = _check_row_projection(got, inp["k_cache"][b, :n, h, :], inp["P"][h], w, kps)
        kp[b, h, :n] = to_dev(kp_ref[b, h])

    # (2) one benchmark step (jssa_decode_step): append the new token at
    # T_b - 1 and decode, in the decode's launches
    kn, vn = _new_token(w, w.seed + 7)
    pos = to_dev(pos_h)
    kn_d, vn_d = to_dev(kn), None if w.mla else to_dev(vn)
    ws = J.workspace(desc, J.OP_DECODE)
    out = torch.empty((B, w.n_q_heads, w.d_v), device=dev)
    lse = torch.empty((B, w.n_q_heads), device=dev)
    J.decode_step(desc, kn_d, vn_d, pos, q, P, kp, K, V, seq, out, lse, ws)
    torch.cuda.synchronize()
    o_bench, l_bench = to_host(out).copy(), to_host(lse).copy()
    # the same step again (the same row re-appended) with the index lists
    # exported, and the plain decode: the same outputs
    idx = torch.full((B, Hkv, w.topk + w.window), -1, dtype=torch.int32, device=dev)
    n_sel = torch.zeros((B, Hkv), dtype=torch.int32, device=dev)
    J.decode_step(desc, kn_d, vn_d, pos, q, P, kp, K, V, seq, out, lse, ws, idx_out=idx, n_sel_out=n_sel)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(out), o_bench) and np.array_equal(to_host(lse), l_bench)
    J.decode(desc, q, P, kp, K, V, seq, out, lse, ws)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(out), o_bench) and np.array_equal(to_host(lse), l_bench)
    status = to_host(J.workspace_status(ws, clear=False))
    gi, gn = to_host(idx), to_host(n_sel)
    _check_structure(gi, gn, L, w)
    assert np.isfinite(o_bench).all() and np.isfinite(l_bench).all()

    # (3) the oracle on each sampled row, with the appended token in its cache
    k_host = inp["k_cache"]
    v_host = k_host[..., :w.d_v] if w.mla else inp["v_cache"]
    for b in range(B):
        k_host[b, pos_h[b]] = kn[b, 0]
        if not w.mla:
            v_host[b, pos_h[b]] = vn[b, 0]
    for b, h in samples:
        n, t = int(L[b]), int(pos_h[b])
        assert np.array_equal(to_host(K[b, t]), kn[b, 0])
        kp_row = np.zeros((T, r), np.uint8 if kps == "fp8" else np.uint16)
        kp_row[:n] = kp_ref[b, h]
        kp_row[t] = _check_row_projection(to_host(kp[b, h, t:t + 1]), k_host[b, t:t + 1, h, :],
                                          inp["P"][h], w, kps)
        hs = slice(h * G, (h + 1) * G)
        qs = inp["q"][b:b + 1, hs]
        s64, n_cand = O.subspace_scores(qs, inp["P"][h:h + 1], kp_row[None, None], L[b:b + 1], w.window,
                                        "max" if reduce == J.REDUCE_MAX else "mean")
        check_sets_within_tolerance(gi[b:b + 1, h:h + 1], gn[b:b + 1, h:h + 1], s64, n_cand, L[b:b + 1],
                                    w.topk, w.window)
        ref, ref_lse = O.attention(qs, k_host[b:b + 1, :, h:h + 1], v_host[b:b + 1, :, h:h + 1],
                                   np.where(gi[b:b + 1, h:h + 1] < 0, 0, gi[b:b + 1, h:h + 1]), gn[b:b + 1, h:h + 1], w.scale)
        got_o, got_l = o_bench[b:b + 1, hs], l_bench[b:b + 1, hs]
        assert rel_l2(got_o, ref) <= ATT_TOL, (b, h, rel_l2(got_o, ref))
        assert np.abs(got_l - ref_lse).max() <= 1e-4 * max(1.0, np.abs(ref_lse).max()), (b, h)
    return status


def test_full_ctx128k_step():
    """Every (sequence, KV head) row against the oracle."""
    w = WORKLOADS["ctx128k"]
    st = _run_full(w, [(b, h) for b in range(w.batch) for h in range(w.n_kv_heads)])
    assert st[J.STATUS_GLOBAL_CUT] == 0


def test_full_ctx128k_step_fp8_keys():
    """The same step with the FP8 E4M3 projected-key cache (the bench's --kp fp8)."""
    _run_full(WORKLOADS["ctx128k"], _eight(WORKLOADS["ctx128k"]), kp_dtype=J.FP8_E4M3)


def test_full_mla_step():
    """All eight sequences (one latent row per sequence)."""
    _run_full(WORKLOADS["mla"], [(b, 0) for b in range(WORKLOADS["mla"].batch)])


def test_full_ctx128k_step_k8192():
    """The budget swept up to k = 8192: about 13,000 tokens pass the sampled
    threshold (about 100 per score tile, read two slot groups at a time); the
    selection holds up to 16,384 in shared memory, so nearly every row is cut
    there (a row past that takes the global cut, covered on its own)."""
    w = scaled(WORKLOADS["ctx128k"], topk=8192)
    st = _run_full(w, _eight(w))
    assert st[J.STATUS_GLOBAL_CUT] <= 3 * w.batch * w.n_kv_heads // 4, st  # the helper decodes three times


def test_full_ctx128k_step_k512():
    """The budget swept down to k = 512."""
    w = scaled(WORKLOADS["ctx128k"], topk=512)
    _run_full(w, _eight(w))


def test_full_hybrid_ragged_step():
    """The hybrid workload at full size: 16 sequences of 8K..128K tokens, the
    last 512 always attended, k = 2048 of the rest.  Whole score workgroups per
    row would give a 128K row's runs 16 tiles against an even share of 14, so
    the rows' tiles are laid end to end and split into equal contiguous ranges
    (some workgroups score the end of one row and the start of the next); the
    new token is the last candidate of each sequence (W + 1 from the end), in
    the last tile of its row.  Checked: two KV heads of every sequence."""
    w = WORKLOADS["hybrid_ragged"]
    st = _run_full(w, [(b, h) for b in range(w.batch) for h in (b % 8, (b + 3) % 8)],
                   pos_of=lambda L: L - w.window - 1)
    assert st[J.STATUS_RANGE_SPLIT] > 0, st  # ranges across rows
