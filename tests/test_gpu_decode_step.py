"""GPU tests of the whole decode step in one call (``jssa_decode_step``: append
the new token, then the decode) against the two calls it stands for
(``jssa_append_kv`` with one token, then ``jssa_decode``) on copies of the same
caches.

In the fused build the append runs inside the scan launch and the scan
re-scores the step that holds the new token, so the cases put the token where
that matters: early in a row (inside the range of the row's first score
workgroup), near the end of the candidates (the last tile of the row's last
score workgroup; ranges that cross rows, with the new token in every
sequence, are in test_gpu_select_paths.py, and the ragged split in the
full-size hybrid step), in the trailing window, past the cache (not
written), and mixed over the batch.  The new key is either a needle (aligned
with its query head's projection and long: selected if it is scored from the
stored row) or a zero row written over a planted needle (selected only if a
stale projected row were scored).  Everything is compared bit for bit: the
caches, the index lists, the outputs and the log-sum-exp values.  In the MLA
layout (MAX) the step's first launch appends the new latent rows and projects
the queries together; the two MLA cases take both of its shapes (rank 64 with
64 heads, rank 32 with 128 heads)."""
import numpy as np
import pytest
import torch

import token_level_sparse_dim_amd as J
from synth import WORKLOADS, generate, scaled, to_bf16_bits

from _gpu_helpers import desc_for, to_dev, to_host

pytestmark = pytest.mark.gpu

CASES = {
    "tiny": WORKLOADS["tiny"],
    "llama": scaled(WORKLOADS["llama8b_32k"], batch=4, t_max=10000, topk=512),
    "128k": scaled(WORKLOADS["ctx128k"], batch=2, t_max=20000, topk=2048),
    "hybrid": scaled(WORKLOADS["hybrid_ragged"], batch=4, t_max=12000, t_min=3000, topk=256),
    "g1r64": scaled(WORKLOADS["llama8b_32k"], batch=2, n_q_heads=4, n_kv_heads=4, rank=64, t_max=6000,
                    topk=100, n_needles=8),
    "g2f32": scaled(WORKLOADS["tiny"], batch=4, n_q_heads=4, n_kv_heads=2, d_k=128, d_v=128, rank=32,
                    t_max=4500, topk=200, window=64),
    "d64bf16": scaled(WORKLOADS["llama8b_32k"], batch=4, d_k=64, d_v=64, rank=16, t_max=7000, topk=300),
    "staged": scaled(WORKLOADS["llama8b_32k"], batch=2, n_q_heads=16, n_kv_heads=8, t_max=5000,
                     topk=128),  # G = 2 in bf16: no fused build
    "mla": scaled(WORKLOADS["mla"], batch=2, n_q_heads=64, t_max=6000, topk=256, n_needles=8),
    # 128 heads at rank 32: the step's first launch with two coordinate tiles
    # per M-tile and an odd batch (the projection waves end mid-workgroup)
    "mla_r32": scaled(WORKLOADS["mla"], batch=3, rank=32, t_max=5000, topk=200, n_needles=8),
}
WHERE = ["early", "late", "last", "mixed"]
_CACHE = {}


def _inputs(w):
    if w not in _CACHE:
        _CACHE[w] = generate(w)
    return _CACHE[w]


def _f32(w, x):
    return (x.astype(np.uint32) << 16).view(np.float32) if w.dtype == "bf16" else x.astype(np.float32)


def _store(w, x):
    return to_bf16_bits(x) if w.dtype == "bf16" else np.ascontiguousarray(x, np.float32)


def _positions(w, L, where):
    """pos[b]: early = a seventh into the candidates, late = just before the
    window (the last candidate tiles), last = T_b - 1, mixed = the three and
    t_max (past the cache) in turn over the batch."""
    n_cand = np.maximum(L - w.window, 0)
    early = np.maximum(n_cand // 7, 0)
    late = np.maximum(n_cand - 1 - np.minimum(3, n_cand - 1), 0)
    last = L - 1
    if where == "early":
        return early
    if where == "late":
        return late
    if where == "last":
        return last
    choice = [early, late, last, np.full_like(L, w.t_max)]
    return np.array([choice[b % 4][b] for b in range(w.batch)])


def _needles(w, inp, pos, sign):
    """New key rows.  sign = +1: the needle c P P^T q / |P^T q| for the KV
    head's first query head q (MLA: query head 0), whose subspace score c
    |P^T q| is 16 times the spread of a random key's score there, so it
    outranks every other token of the row; sign = -1: zero rows written over
    that same needle planted at pos first (a zero key scores exactly 0, below
    the k-th score when the row has four times more candidates than the
    budget; the stale projected row would rank first).  Values are random."""
    q = _f32(w, inp["q"])
    G = w.group
    kf = _f32(w, inp["k_cache"][:, :256])  # the keys' typical norm
    c = 16.0 * float(np.sqrt((kf.astype(np.float64) ** 2).sum(-1).mean()))
    needle = np.zeros((w.batch, 1, w.n_kv_heads, w.d_k), np.float32)
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            qh = q[b, 0 if w.mla else h * G].astype(np.float64)
            Ph = inp["P"][h].astype(np.float64)
            u = Ph @ (Ph.T @ qh)
            needle[b, 0, h] = c * u / np.linalg.norm(Ph.T @ qh)
    k_cache = inp["k_cache"].copy()
    kn = needle
    if sign < 0:
        for b in range(w.batch):
            if pos[b] < w.t_max:
                k_cache[b, pos[b]] = _store(w, needle[b, 0])
        kn = np.zeros_like(needle)
    rng = np.random.default_rng(w.seed + 11)
    vn = None if w.mla else rng.standard_normal((w.batch, 1, w.n_kv_heads, w.d_v)).astype(np.float32)
    return _store(w, kn), None if vn is None else _store(w, vn), k_cache


def _state(w, desc, inp, k_cache):
    """Device copies of the caches, the scoring cache projected on the GPU."""
    K = to_dev(k_cache)
    V = None if w.mla else to_dev(inp["v_cache"])
    tdt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    kp = torch.empty((w.batch, w.n_kv_heads, w.t_max, w.rank), dtype=tdt, device="cuda")
    J.append_projection(desc, w.t_max, torch.zeros(w.batch, dtype=torch.int32, device="cuda"),
                        to_dev(inp["P"]), K, kp)
    return K, V, kp


def _outputs(w):
    return (torch.empty((w.batch, w.n_q_heads, w.d_v), device="cuda"),
            torch.empty((w.batch, w.n_q_heads), device="cuda"),
            torch.full((w.batch, w.n_kv_heads, w.topk + w.window), -1, dtype=torch.int32, device="cuda"),
            torch.zeros((w.batch, w.n_kv_heads), dtype=torch.int32, device="cuda"))


def _compare(w, where, sign, reduce=J.REDUCE_MAX, events=False):
    inp = _inputs(w)
    desc = desc_for(w, reduce=reduce)
    L = inp["seq_lens"].astype(np.int64)
    pos = _positions(w, L, where)
    kn, vn, k_cache = _needles(w, inp, pos, sign)
    q, P, seq = to_dev(inp["q"]), to_dev(inp["P"]), to_dev(inp["seq_lens"])
    pos_d = to_dev(pos.astype(np.int32))
    kn_d, vn_d = to_dev(kn), None if vn is None else to_dev(vn)

    # the two calls
    K1, V1, kp1 = _state(w, desc, inp, k_cache)
    out1, lse1, idx1, n1 = _outputs(w)
    ws1 = J.workspace(desc, J.OP_DECODE)
    J.append_kv(desc, kn_d, vn_d, pos_d, P, K1, V1, kp1)
    J.decode(desc, q, P, kp1, K1, V1, seq, out1, lse1, ws1, idx_out=idx1, n_sel_out=n1)
    # the one call
    K2, V2, kp2 = _state(w, desc, inp, k_cache)
    out2, lse2, idx2, n2 = _outputs(w)
    ws2 = J.workspace(desc, J.OP_DECODE)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)] if events else None
    J.decode_step(desc, kn_d, vn_d, pos_d, q, P, kp2, K2, V2, seq, out2, lse2, ws2, idx_out=idx2,
                  n_sel_out=n2, events=ev)
    torch.cuda.synchronize()

    assert np.array_equal(to_host(kp2), to_host(kp1))
    assert np.array_equal(to_host(K2), to_host(K1))
    if not w.mla:
        assert np.array_equal(to_host(V2), to_host(V1))
    gi, gn = to_host(idx2), to_host(n2)
    assert np.array_equal(gn, to_host(n1))
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            assert np.array_equal(gi[b, h, :gn[b, h]], to_host(idx1)[b, h, :gn[b, h]]), (b, h)
    assert np.array_equal(to_host(out2), to_host(out1))
    assert np.array_equal(to_host(lse2), to_host(lse1))

    # where the token at pos is a candidate of its row: the needle is
    # selected, the zero row written over a needle is not (max reduction)
    n_cand = np.maximum(L - w.window, 0)
    hit = 0
    for b in range(w.batch if reduce == J.REDUCE_MAX else 0):
        if pos[b] >= n_cand[b] or pos[b] >= w.t_max or n_cand[b] <= (w.topk if sign > 0 else 4 * w.topk):
            continue
        for h in range(w.n_kv_heads):
            sel = gi[b, h, :gn[b, h]]
            assert (pos[b] in sel) == (sign > 0), (b, h, int(pos[b]), sign)
            hit += 1
    return hit


@pytest.mark.parametrize("sign", [1, -1], ids=["needle", "overwrite"])
@pytest.mark.parametrize("where", WHERE)
@pytest.mark.parametrize("name", list(CASES))
def test_decode_step_equals_append_then_decode(name, where, sign):
    w = CASES[name]
    hit = _compare(w, where, sign)
    if where in ("early", "late"):
        assert hit > 0  # the case exercises a scored token


@pytest.mark.parametrize("name", ["128k", "g1r64", "g2f32"])
def test_decode_step_mean_reduction_and_events(name):
    _compare(CASES[name], "mixed", 1, reduce=J.REDUCE_MEAN, events=True)


def test_decode_step_repeated_calls():
    """The benchmark's pattern: the same step again on the updated caches and
    the same workspace (the new row is rewritten with the same values)."""
    w = CASES["128k"]
    inp = _inputs(w)
    desc = desc_for(w)
    L = inp["seq_lens"].astype(np.int64)
    pos = _positions(w, L, "late")
    kn, vn, k_cache = _needles(w, inp, pos, 1)
    q, P, seq = to_dev(inp["q"]), to_dev(inp["P"]), to_dev(inp["seq_lens"])
    K, V, kp = _state(w, desc, inp, k_cache)
    out, lse, idx, n = _outputs(w)
    ws = J.workspace(desc, J.OP_DECODE)
    res = []
    for _ in range(3):
        J.decode_step(desc, to_dev(kn), to_dev(vn), to_dev(pos.astype(np.int32)), q, P, kp, K, V, seq, out, lse,
                      ws, idx_out=idx, n_sel_out=n)
        torch.cuda.synchronize()
        res.append((to_host(out).copy(), to_host(lse).copy(), to_host(idx).copy(), to_host(n).copy()))
    for r in res[1:]:
        for a, b in zip(r, res[0]):
            assert np.array_equal(a, b)
