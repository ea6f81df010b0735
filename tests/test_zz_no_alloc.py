"""GPU test of jssa_decode_step_static, the allocation-free variant of
jssa_decode_step: through the C ABI, on copies of the same caches, it must give
exactly what jssa_decode_step gives with a fresh workspace (the appended cache
rows, the index lists, the outputs and the log-sum-exp values, bit for bit),
on two calls in a row, the second with a smaller input (fewer rows, shorter
caches) that lands on the static scratch the first call left behind."""
import dataclasses

import numpy as np
import pytest
import torch

import token_level_sparse_dim_amd as J
from synth import WORKLOADS, generate, scaled, to_bf16_bits

from _gpu_helpers import desc_for, oracle_kp, to_dev, to_host

pytestmark = pytest.mark.gpu

FIRST = scaled(WORKLOADS["hybrid_ragged"], batch=6, t_max=40000, t_min=20000, topk=2048)
SECOND = scaled(WORKLOADS["ctx128k"], batch=1, n_kv_heads=4, n_q_heads=16, t_max=9000, topk=512)


def _step_both(w, seed):
    inp = generate(w)
    desc = desc_for(w)
    kp_h = oracle_kp(inp, desc)
    rng = np.random.default_rng(seed)
    kn = to_dev(to_bf16_bits(rng.standard_normal((w.batch, 1, w.n_kv_heads, w.d_k)).astype(np.float32)))
    vn = to_dev(to_bf16_bits(rng.standard_normal((w.batch, 1, w.n_kv_heads, w.d_v)).astype(np.float32)))
    L = inp["seq_lens"]
    pos = to_dev(np.maximum(L - w.window - 1 - (np.arange(w.batch) % 3) * 977, 0).astype(np.int32))
    q, P, seq = to_dev(inp["q"]), to_dev(inp["P"]), to_dev(inp["seq_lens"])
    res = []
    for static in (False, True):
        K, V, KP = to_dev(inp["k_cache"]), to_dev(inp["v_cache"]), to_dev(kp_h)
        out = torch.empty((w.batch, w.n_q_heads, w.d_v), device="cuda")
        lse = torch.empty((w.batch, w.n_q_heads), device="cuda")
        idx = torch.full((w.batch, w.n_kv_heads, w.topk + w.window), -1, dtype=torch.int32, device="cuda")
        n_sel = torch.zeros((w.batch, w.n_kv_heads), dtype=torch.int32, device="cuda")
        if static:
            J.decode_step_static(desc, kn, vn, pos, q, P, KP, K, V, seq, out, lse, idx_out=idx, n_sel_out=n_sel)
        else:
            J.decode_step(desc, kn, vn, pos, q, P, KP, K, V, seq, out, lse, J.workspace(desc, J.OP_DECODE),
                          idx_out=idx, n_sel_out=n_sel)
        torch.cuda.synchronize()
        res.append([to_host(x) for x in (K, V, KP, idx, n_sel, out, lse)])
        del K, V, KP
    for a, b, name in zip(res[0], res[1], ("k_cache", "v_cache", "kp_cache", "idx", "n_sel", "out", "lse")):
        assert np.array_equal(a, b), (w.name, name)
    return res[1]


def test_static_step_equals_workspace_step_twice():
    print("static decode step: first call", FIRST, flush=True)
    first = _step_both(FIRST, 3)
    assert (first[4] > 0).all() and np.isfinite(first[5]).all()
    print("static decode step: second, smaller call", SECOND, flush=True)
    second = _step_both(SECOND, 4)
    assert (second[4] > 0).all() and np.isfinite(second[5]).all()


def test_static_step_rejects_what_it_does_not_hold():
    w = FIRST
    base = desc_for(w)
    big = dataclasses.replace(base, batch=64, t_max=1 << 20)  # 512 rows x 1M tokens of candidate slots
    mla = desc_for(WORKLOADS["mla"])
    d = torch.zeros(16, dtype=torch.int32, device="cuda")
    p = d.data_ptr()
    lib = J.lib()
    args = (p,) * 13 + (None,)
    assert lib.jssa_decode_step_static(big.c(), *args) == -6  # JSSA_ERR_TOO_LARGE
    assert lib.jssa_decode_step_static(mla.c(), *args) == -2  # no fused build: unsupported
