"""The whole decode step captured in a HIP graph and replayed: every launch of
``jssa_decode_step`` only enqueues kernels on the caller's stream (no
allocation, no memset node, counters that reset themselves), so a captured
step replays to the eager result, replay after replay, with other eager
decode work and synchronisations in between."""
import numpy as np
import pytest
import torch

import token_level_sparse_dim_amd as J
from synth import WORKLOADS, generate, scaled, to_bf16_bits

from _gpu_helpers import desc_for, to_dev, to_host

pytestmark = pytest.mark.gpu

CASES = {
    "128k": (scaled(WORKLOADS["ctx128k"], batch=2, t_max=20000, topk=2048), J.BF16),
    "128k_fp8": (scaled(WORKLOADS["ctx128k"], batch=2, t_max=20000, topk=2048), J.FP8_E4M3),
    "hybrid": (scaled(WORKLOADS["hybrid_ragged"], batch=3, t_max=12000, t_min=3000, topk=256), J.BF16),
    "mla": (scaled(WORKLOADS["mla"], batch=2, t_max=6000, topk=256, n_needles=8), J.BF16),
}


class _Step:
    """Caches, inputs and outputs of one decode step, all device-resident."""

    def __init__(self, w, kp_dtype, seed):
        inp = generate(w, seed=seed)
        self.w = w
        self.desc = desc_for(w, kp_dtype=kp_dtype)
        self.q, self.P, self.seq = to_dev(inp["q"]), to_dev(inp["P"]), to_dev(inp["seq_lens"])
        self.K = to_dev(inp["k_cache"])
        self.V = None if w.mla else to_dev(inp["v_cache"])
        kdt = torch.uint8 if kp_dtype == J.FP8_E4M3 else torch.bfloat16
        self.kp = torch.empty((w.batch, w.n_kv_heads, w.t_max, w.rank), dtype=kdt, device="cuda")
        J.append_projection(self.desc, w.t_max, torch.zeros(w.batch, dtype=torch.int32, device="cuda"),
                            self.P, self.K, self.kp)
        rng = np.random.default_rng(seed + 1)
        self.kn = to_dev(to_bf16_bits(rng.standard_normal((w.batch, 1, w.n_kv_heads, w.d_k)).astype(np.float32)))
        self.vn = None if w.mla else to_dev(
            to_bf16_bits(rng.standard_normal((w.batch, 1, w.n_kv_heads, w.d_v)).astype(np.float32)))
        self.pos = (self.seq - 1).contiguous()
        self.ws = J.workspace(self.desc, J.OP_DECODE)
        self.out = torch.empty((w.batch, w.n_q_heads, w.d_v), device="cuda")
        self.lse = torch.empty((w.batch, w.n_q_heads), device="cuda")
        self.idx = torch.full((w.batch, w.n_kv_heads, w.topk + w.window), -1, dtype=torch.int32, device="cuda")
        self.n_sel = torch.zeros((w.batch, w.n_kv_heads), dtype=torch.int32, device="cuda")

    def run(self):
        J.decode_step(self.desc, self.kn, self.vn, self.pos, self.q, self.P, self.kp, self.K, self.V, self.seq,
                      self.out, self.lse, self.ws, idx_out=self.idx, n_sel_out=self.n_sel)

    def result(self):
        return [to_host(t).copy() for t in (self.out, self.lse, self.idx, self.n_sel, self.kp)]


@pytest.mark.parametrize("name", list(CASES))
def test_decode_step_graph_replays_equal_eager(name):
    w, kpt = CASES[name]
    st = _Step(w, kpt, w.seed)
    other = _Step(w, kpt, w.seed + 100)  # eager work between the replays
    st.run()  # eager: the reference (and every host-side cache warm)
    other.run()
    torch.cuda.synchronize()
    ref = st.result()
    for t in (st.out, st.lse):
        t.fill_(float("nan"))
    st.idx.fill_(-1)
    st.n_sel.fill_(0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            st.run()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(4):
        g.replay()
        torch.cuda.synchronize()
        got = st.result()
        for a, b in zip(got[:2], ref[:2]):
            assert np.array_equal(a, b, equal_nan=True), rep
        gn = got[3]
        assert np.array_equal(gn, ref[3]), rep
        for b_ in range(w.batch):
            for h in range(w.n_kv_heads):
                assert np.array_equal(got[2][b_, h, :gn[b_, h]], ref[2][b_, h, :gn[b_, h]]), (rep, b_, h)
        assert np.array_equal(got[4], ref[4]), rep
        other.run()  # eager decode work on other buffers and workspace between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("name", ["128k", "hybrid"])
def test_layer_stack_graph_replays_equal_eager(name):
    """Three layers in one graph: an indexer layer (``jssa_decode_step``), a
    layer reusing its lists (``jssa_reuse_step``), another indexer layer;
    each with its own query and caches, one workspace for all."""
    w, kpt = CASES[name]
    layers = [_Step(w, kpt, w.seed + 10 * l) for l in range(3)]
    other = _Step(w, kpt, w.seed + 100)
    ws = layers[0].ws

    def stack():
        for l, y in enumerate(layers):
            if l % 2 == 0:
                J.decode_step(y.desc, y.kn, y.vn, y.pos, y.q, y.P, y.kp, y.K, y.V, y.seq, y.out, y.lse, ws,
                              idx_out=y.idx, n_sel_out=y.n_sel)
            else:
                src = layers[l - 1]
                J.reuse_step(y.desc, y.kn, y.vn, y.pos, y.q, y.K, y.V, src.idx, src.n_sel, y.out, y.lse, ws)

    stack()
    other.run()
    torch.cuda.synchronize()
    ref = [y.result() for y in layers]
    for y in layers:
        y.out.fill_(float("nan"))
        y.lse.fill_(float("nan"))
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            stack()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(4):
        g.replay()
        torch.cuda.synchronize()
        for l, y in enumerate(layers):
            got = y.result()
            assert np.array_equal(got[0], ref[l][0], equal_nan=True), (rep, l)
            assert np.array_equal(got[1], ref[l][1], equal_nan=True), (rep, l)
            if l % 2 == 0:
                assert np.array_equal(got[3], ref[l][3]), (rep, l)
            assert np.array_equal(got[4], ref[l][4]), (rep, l)
        other.run()
        torch.cuda.synchronize()
