"""GPU tests of the layer that reuses an indexer layer's selection
(``jssa_reuse_step``; JSSA summary appendix C: selection only at indexer
layers, the adjacent layers reuse the indices).  A two-layer step: layer 0
is an indexer layer (``jssa_decode_step``: append, score, select, attend),
layer 1 has its own query and caches and no scoring cache; it writes its new
K/V rows (bit for bit the oracle's) and attends over layer 0's lists, to the
oracle's attention of its own rows at those positions.  With no new rows the
call is the indexed attention."""
import numpy as np
import pytest
import torch

import token_level_sparse_dim_amd as J
from oracle import jssa_oracle as O
from synth import WORKLOADS, generate, scaled, to_bf16_bits

from _gpu_helpers import desc_for, oracle_kp, rel_l2, to_dev, to_host

pytestmark = pytest.mark.gpu

CASES = {
    "128k": (scaled(WORKLOADS["ctx128k"], batch=2, t_max=20000, topk=2048), J.BF16),
    "128k_fp8": (scaled(WORKLOADS["ctx128k"], batch=2, t_max=20000, topk=2048), J.FP8_E4M3),
    "hybrid": (scaled(WORKLOADS["hybrid_ragged"], batch=4, t_max=12000, t_min=300, topk=256), J.BF16),
    "staged": (scaled(WORKLOADS["llama8b_32k"], batch=2, n_q_heads=16, n_kv_heads=8, t_max=5000, topk=128),
               J.BF16),  # G = 2 in bf16: the stand-alone attention
    "tiny_f32": (WORKLOADS["tiny"], None),
    "mla": (scaled(WORKLOADS["mla"], batch=2, n_q_heads=64, t_max=6000, topk=256, n_needles=8), J.BF16),
}


def _rows(w, rng, n_heads, d):
    x = rng.standard_normal((w.batch, 1, n_heads, d)).astype(np.float32)
    return to_bf16_bits(x) if w.dtype == "bf16" else x


@pytest.mark.parametrize("name", list(CASES))
def test_reuse_layer_matches_oracle(name):
    w, kpt = CASES[name]
    l0 = generate(w)
    l1 = generate(w, seed=w.seed + 7)  # another layer: its own query and caches
    seq = l0["seq_lens"].copy()
    if name == "hybrid":
        seq[1] = 0  # an empty sequence: nothing appended (pos -1), nothing attended
        seq[2] = w.window + 50
    pos = (seq.astype(np.int64) - 1).astype(np.int32)
    desc = desc_for(w, kp_dtype=kpt) if kpt is not None else desc_for(w)
    rng = np.random.default_rng(11)
    kn0, kn1 = (_rows(w, rng, w.n_kv_heads, w.d_k) for _ in range(2))
    vn0 = vn1 = None
    if not w.mla:
        vn0, vn1 = (_rows(w, rng, w.n_kv_heads, w.d_v) for _ in range(2))
    S, P, pos_d = to_dev(seq), to_dev(l0["P"]), to_dev(pos)
    kp0 = to_dev(oracle_kp({**l0, "seq_lens": seq}, desc))
    K0, K1 = to_dev(l0["k_cache"]), to_dev(l1["k_cache"])
    V0 = None if w.mla else to_dev(l0["v_cache"])
    V1 = None if w.mla else to_dev(l1["v_cache"])
    idx = torch.full((w.batch, w.n_kv_heads, w.topk + w.window), -1, dtype=torch.int32, device="cuda")
    n_sel = torch.zeros((w.batch, w.n_kv_heads), dtype=torch.int32, device="cuda")
    outs = [torch.empty((w.batch, w.n_q_heads, w.d_v), device="cuda") for _ in range(3)]
    lses = [torch.empty((w.batch, w.n_q_heads), device="cuda") for _ in range(3)]
    ws = J.workspace(desc, J.OP_DECODE)
    J.decode_step(desc, to_dev(kn0), None if w.mla else to_dev(vn0), pos_d, to_dev(l0["q"]), P, kp0, K0, V0, S,
                  outs[0], lses[0], ws, idx_out=idx, n_sel_out=n_sel)
    q1 = to_dev(l1["q"])
    J.reuse_step(desc, to_dev(kn1), None if w.mla else to_dev(vn1), pos_d, q1, K1, V1, idx, n_sel,
                 outs[1], lses[1], ws)
    torch.cuda.synchronize()
    # the new rows, bit for bit
    k1 = O.write_new_rows(l1["k_cache"], kn1, pos)
    assert np.array_equal(to_host(K1), k1)
    v1 = None
    if not w.mla:
        v1 = O.write_new_rows(l1["v_cache"], vn1, pos)
        assert np.array_equal(to_host(V1), v1)
    else:
        v1 = k1[..., :w.d_v]
    # the attention over layer 0's lists
    gi, gn = to_host(idx), to_host(n_sel)
    assert np.array_equal(gn, np.array([[O.n_selected(int(t), w.topk, w.window)] * w.n_kv_heads for t in seq]))
    ref, ref_lse = O.attention(l1["q"], k1, v1, np.where(gi < 0, 0, gi), gn, w.scale)
    tol = 1e-5 if w.dtype == "f32" else 2e-3
    assert rel_l2(to_host(outs[1]), ref) <= tol
    fin = np.isfinite(ref_lse)
    got_lse = to_host(lses[1])
    assert np.array_equal(np.isfinite(got_lse), fin)
    assert np.abs(got_lse[fin] - ref_lse[fin]).max(initial=0) <= 1e-4 * max(1.0, np.abs(ref_lse[fin]).max(initial=0))
    if name == "hybrid":
        assert (to_host(outs[1])[1] == 0).all()
    # no new rows: the call is the indexed attention on the (updated) caches, bit for bit
    J.reuse_step(desc, None, None, None, q1, K1, V1, idx, n_sel, outs[2], lses[2], ws)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(outs[2]), to_host(outs[1]))
    assert np.array_equal(to_host(lses[2]), to_host(lses[1]), equal_nan=True)
