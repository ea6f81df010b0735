"""GPU tests of the gather-then-attend baseline (JSSA summary section 2.2 and
Figure 2(b); section 4.7 compares it with gather-free execution on the same
selected tokens): ``jssa_gather_kv`` packs the selected rows, bit for bit
equal to the oracle's gather, and the dense decode over the packed rows is
the indexed attention over the lists, within the attention tolerance of both
the gather-free kernel and the oracle."""
import numpy as np
import pytest
import torch

import token_level_sparse_dim_amd as J
from oracle import jssa_oracle as O
from synth import WORKLOADS, generate, scaled

from _gpu_helpers import desc_for, rel_l2, to_dev, to_host

pytestmark = pytest.mark.gpu

CASES = {
    "tiny": WORKLOADS["tiny"],
    "llama": scaled(WORKLOADS["llama8b_32k"], batch=2, t_max=6000, topk=512),
    "hybrid": scaled(WORKLOADS["hybrid_ragged"], batch=3, t_max=8000, t_min=300, topk=256),
    "mla": scaled(WORKLOADS["mla"], batch=2, t_max=4000, topk=256, n_needles=8),
}
_CACHE = {}


def inputs(w):
    if w not in _CACHE:
        _CACHE[w] = generate(w)
    return _CACHE[w]


def _lists(w, inp, rng, unsorted):
    """Valid index lists with the decode's counts: n_sel = min(W, T_b) +
    min(k, T_b - W) per sequence, entries drawn from [0, T_b) (repeats
    allowed, sorted unless `unsorted`)."""
    S = w.topk + w.window
    L = inp["seq_lens"].astype(np.int64)
    idx = np.full((w.batch, w.n_kv_heads, S), -1, np.int32)
    n_sel = np.zeros((w.batch, w.n_kv_heads), np.int32)
    for b in range(w.batch):
        n = O.n_selected(int(L[b]), w.topk, w.window)
        for h in range(w.n_kv_heads):
            v = rng.integers(0, int(L[b]), size=n).astype(np.int32)
            idx[b, h, :n] = v if unsorted else np.sort(v)
            n_sel[b, h] = n
    return idx, n_sel


def _packed_desc(w, S):
    return desc_for(w, t_max=S, topk=S, window=0)


@pytest.mark.parametrize("unsorted", [False, True], ids=["sorted", "unsorted"])
@pytest.mark.parametrize("name", list(CASES))
def test_gather_then_dense_equals_indexed_attention(name, unsorted):
    w = CASES[name]
    inp = inputs(w)
    desc = desc_for(w)
    rng = np.random.default_rng(5 + unsorted)
    idx, n_sel = _lists(w, inp, rng, unsorted)
    S = w.topk + w.window
    kv = torch.float32 if w.dtype == "f32" else torch.bfloat16
    K = to_dev(inp["k_cache"])
    V = None if w.mla else to_dev(inp["v_cache"])
    Kg = torch.zeros((w.batch, S, w.n_kv_heads, w.d_k), dtype=kv, device="cuda")
    Vg = None if w.mla else torch.zeros((w.batch, S, w.n_kv_heads, w.d_v), dtype=kv, device="cuda")
    lens = torch.full((w.batch,), -7, dtype=torch.int32, device="cuda")
    J.gather_kv(desc, K, V, to_dev(idx), to_dev(n_sel), Kg, Vg, lens)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(lens), n_sel[:, 0])
    assert np.array_equal(to_host(Kg), O.gather_rows(inp["k_cache"], idx, n_sel))
    if not w.mla:
        assert np.array_equal(to_host(Vg), O.gather_rows(inp["v_cache"], idx, n_sel))

    # attention: gather-free on the lists vs dense on the packed rows
    q = to_dev(inp["q"])
    out_i = torch.empty((w.batch, w.n_q_heads, w.d_v), device="cuda")
    lse_i = torch.empty((w.batch, w.n_q_heads), device="cuda")
    J.indexed_attn(desc, q, K, V, to_dev(idx), to_dev(n_sel), out_i, lse_i, J.workspace(desc, J.OP_ATTN))
    pdesc = _packed_desc(w, S)
    out_g = torch.empty_like(out_i)
    lse_g = torch.empty_like(lse_i)
    J.dense_decode(pdesc, q, Kg, Vg, lens, out_g, lse_g, J.workspace(pdesc, J.OP_DENSE))
    torch.cuda.synchronize()
    v_host = inp["k_cache"][..., :w.d_v] if w.mla else inp["v_cache"]
    ref, ref_lse = O.attention(inp["q"], inp["k_cache"], v_host, np.where(idx < 0, 0, idx), n_sel, w.scale)
    tol = 1e-5 if w.dtype == "f32" else 2e-3
    oi, og = to_host(out_i), to_host(out_g)
    assert rel_l2(og, ref) <= tol and rel_l2(oi, ref) <= tol
    assert rel_l2(og, oi) <= tol
    li, lg = to_host(lse_i), to_host(lse_g)
    assert np.abs(lg - ref_lse).max() <= 1e-4 * max(1.0, np.abs(ref_lse).max())
    assert np.abs(li - lg).max() <= 1e-4 * max(1.0, np.abs(ref_lse).max())


def test_gather_of_decode_selection_and_empty_rows():
    """The lists a decode step produced (ascending, window last) and sequences
    whose list is empty (T_b = 0): nothing packed, dense output 0 and lse -inf,
    as for the indexed attention."""
    w = CASES["hybrid"]
    inp = inputs(w)
    desc = desc_for(w)
    seq = inp["seq_lens"].copy()
    seq[1] = 0
    kp, _ = O.project_keys(inp["k_cache"], inp["P"], seq, "bf16")
    out = torch.empty((w.batch, w.n_q_heads, w.d_v), device="cuda")
    idx = torch.full((w.batch, w.n_kv_heads, w.topk + w.window), -1, dtype=torch.int32, device="cuda")
    n_sel = torch.zeros((w.batch, w.n_kv_heads), dtype=torch.int32, device="cuda")
    K, V, q = to_dev(inp["k_cache"]), to_dev(inp["v_cache"]), to_dev(inp["q"])
    J.decode(desc, q, to_dev(inp["P"]), to_dev(kp), K, V, to_dev(seq), out, None, J.workspace(desc, J.OP_DECODE),
             idx_out=idx, n_sel_out=n_sel)
    S = w.topk + w.window
    Kg = torch.zeros((w.batch, S, w.n_kv_heads, w.d_k), dtype=torch.bfloat16, device="cuda")
    Vg = torch.zeros_like(Kg)
    lens = torch.empty((w.batch,), dtype=torch.int32, device="cuda")
    J.gather_kv(desc, K, V, idx, n_sel, Kg, Vg, lens)
    gi, gn = to_host(idx), to_host(n_sel)
    assert gn[1].sum() == 0 and to_host(lens)[1] == 0
    assert np.array_equal(to_host(Kg), O.gather_rows(inp["k_cache"], gi, gn))
    pdesc = _packed_desc(w, S)
    out_g = torch.empty((w.batch, w.n_q_heads, w.d_v), device="cuda")
    lse_g = torch.empty((w.batch, w.n_q_heads), device="cuda")
    J.dense_decode(pdesc, q, Kg, Vg, lens, out_g, lse_g, J.workspace(pdesc, J.OP_DENSE))
    og, lg = to_host(out_g), to_host(lse_g)
    assert (og[1] == 0).all() and np.isneginf(lg[1]).all()
    ref, _ = O.attention(inp["q"], inp["k_cache"], inp["v_cache"], np.where(gi < 0, 0, gi), gn, w.scale)
    assert rel_l2(og, ref) <= 2e-3
