"""Seeded input generator: determinism and the structure the workloads promise."""
import numpy as np

import synth
from synth import inputs as S


def _small_hybrid():
    return S.scaled(S.WORKLOADS["hybrid_ragged"], batch=3, t_max=4096, t_min=1024, topk=64, window=128)


def test_same_seed_same_bytes_and_thread_count_free(monkeypatch):
    w = S.scaled(S.WORKLOADS["llama8b_32k"], batch=2, t_max=2 * S.CHUNK + 100)
    a = S.generate(w)
    monkeypatch.setattr(S, "_threads", lambda: 1)
    b = S.generate(w)
    for key in ("P", "q", "k_cache", "v_cache", "seq_lens", "needles"):
        assert np.array_equal(a[key], b[key]), key
    c = S.generate(w, seed=w.seed + 100)
    assert not np.array_equal(a["k_cache"], c["k_cache"])


def test_basis_is_orthonormal_per_head():
    d = S.generate(S.WORKLOADS["tiny"])
    P = d["P"].astype(np.float64)
    for h in range(P.shape[0]):
        assert np.allclose(P[h].T @ P[h], np.eye(P.shape[2]), atol=1e-6)
    assert not np.allclose(P[0], P[1])


def test_ragged_lengths_needles_and_zero_tail():
    w = _small_hybrid()
    d = S.generate(w)
    L = d["seq_lens"]
    assert ((L >= w.t_min) & (L <= w.t_max)).all()
    for b in range(w.batch):
        assert (d["k_cache"][b, L[b]:] == 0).all()
        for h in range(w.n_kv_heads):
            pos = d["needles"][b, h]
            assert len(set(pos.tolist())) == pos.size
            assert (pos < L[b] - w.window).all()
    # needle positions differ between KV heads
    assert not all(np.array_equal(d["needles"][0, 0], d["needles"][0, h]) for h in range(1, w.n_kv_heads))


def test_bf16_bits_roundtrip():
    x = np.array([1.0, -2.5, 3.140625, 0.0], np.float32)
    assert np.array_equal(synth.bf16_bits_to_f32(synth.to_bf16_bits(x)), x)


def test_mla_has_no_separate_values():
    w = S.scaled(S.WORKLOADS["mla"], batch=1, t_max=2048, n_needles=8)
    d = S.generate(w)
    assert d["v_cache"] is None and d["k_cache"].shape == (1, 2048, 1, 576)
