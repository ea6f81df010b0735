"""Seeded synthetic decode-step inputs for token-level sparse decode attention.

This module only *makes inputs*: the orthonormal scoring basis, the query,
the key/value cache, the per-sequence lengths and the planted "needle"
positions.  It holds none of the method's arithmetic (no key projection, no
scoring, no selection, no attention), so that the CPU oracle and the HIP path
can both consume it without sharing any computation.

Shapes follow the decode step of Joint Subspace Sparse Attention (paperlayer
summary of arXiv 2610.19026, section 3.1 and Figure 1): a GQA KV cache in the
standard ``[B, T, Hkv, d]`` layout, one query token per sequence
``[B, Hq, d]``, and one ``d x r`` orthonormal basis per KV head (section 3.2).
The pages evaluate on LongBench / RULER / PG-19 and real checkpoints, none of
which are available here; these synthetic workloads stand in for them with
the pages' shapes (128K context and a 2,048-token budget, section 4.5;
32-dimensional scoring, section 3.4; BF16 K/V, appendix A.3).

Recipe (all draws from ``numpy.random.PCG64``; every stream is a child of
``SeedSequence(seed)`` spawned in a fixed order, and the bulk streams are
further split into fixed 16,384-token chunks so the result does not depend
on the number of worker threads):

* ``P[h]``: reduced QR (Q factor) of a ``d x r`` standard-normal matrix,
  stored fp32.
* ``A[h]``: ``d x key_rank`` with entries ``N(0, 1/d)``.
* keys: ``K[b,t,h] = A[h] z + 0.1 eps`` with ``z ~ N(0, I_key_rank)`` and
  ``eps ~ N(0, I_d)``.
* values: ``V ~ N(0, 1)``.
* query: ``q[b,hq] = A[hq // G] z_q + 0.1 noise``.
* needles: ``n_needles`` distinct candidate positions per (sequence, KV head);
  needle ``j`` of KV head ``h`` is ``3 q / |q|`` for query head
  ``h*G + (j mod G)`` (MLA: query head ``(2 j) mod Hq``).
* ragged workloads draw ``T_b`` uniformly from ``[t_min, t_max]``.
* bf16 workloads round fp32 to bf16 with round-to-nearest-even (torch's
  conversion) and are returned as ``uint16`` bit patterns.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace

import numpy as np
import torch

CHUNK = 16384  # tokens per independently seeded bulk chunk


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    d_k: int
    d_v: int
    rank: int               # scoring rank r
    t_max: int              # cache capacity and (non-ragged) context length
    topk: int               # budget k
    window: int = 0         # trailing always-attended tokens W
    dtype: str = "bf16"     # 'f32' or 'bf16' (q, K, V and the projected-key cache)
    key_rank: int = 16      # rank of the low-rank part of the keys
    n_needles: int = 32     # planted needles per (sequence, KV head)
    t_min: int | None = None  # ragged lengths drawn from [t_min, t_max]
    mla: bool = False       # one shared latent row per token; V = first d_v columns
    seed: int = 1000

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.d_k))

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2


WORKLOADS: dict[str, Workload] = {
    # tiny fp32 GQA step
    "tiny": Workload("tiny-fp32-gqa", 1, 8, 2, 64, 64, 16, 1024, 64, 0, "f32",
                     key_rank=8, n_needles=4, seed=1001),
    # one Llama-3-8B-shaped layer, 32K context
    "llama8b_32k": Workload("llama3-8b-layer-32k", 8, 32, 8, 128, 128, 32, 32768, 2048,
                            key_rank=16, n_needles=32, seed=1002),
    # 128K long-context decode (the headline workload)
    "ctx128k": Workload("gqa-128k-k2048", 4, 32, 8, 128, 128, 32, 131072, 2048,
                        key_rank=16, n_needles=32, seed=1003),
    # hybrid local/global: trailing window of 512 plus top-k of the rest, ragged batch
    "hybrid_ragged": Workload("hybrid-ragged-w512", 16, 32, 8, 128, 128, 32, 131072, 2048,
                              window=512, key_rank=16, n_needles=32, t_min=8192, seed=1004),
    # MLA-shaped decode: 128 query heads share one 576-wide latent row
    "mla": Workload("mla-128k-k2048", 8, 128, 1, 576, 512, 64, 131072, 2048,
                    key_rank=32, n_needles=64, mla=True, seed=1005),
}


def scaled(w: Workload, **kw) -> Workload:
    """Same structure, different sizes (used for down-scaled parity cases)."""
    return replace(w, **kw)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(u: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp32 values (exact)."""
    return (np.asarray(u, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _store(w: Workload, x: np.ndarray) -> np.ndarray:
    return to_bf16_bits(x) if w.dtype == "bf16" else np.ascontiguousarray(x, dtype=np.float32)


def _load(w: Workload, x: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(x) if w.dtype == "bf16" else x.astype(np.float32)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def generate(w: Workload, seed: int | None = None) -> dict:
    """Generate one decode step's inputs for workload ``w``.

    Returns a dict with
      ``P`` fp32 ``[Hkv, d_k, r]``; ``q`` ``[B, Hq, d_k]``;
      ``k_cache`` ``[B, t_max, Hkv, d_k]``; ``v_cache`` ``[B, t_max, Hkv, d_v]``
      (``None`` for MLA, where V is the first ``d_v`` columns of ``k_cache``);
      ``seq_lens`` int32 ``[B]``; ``needles`` int32 ``[B, Hkv, n_needles]``.
    q/K/V are uint16 bf16 bit patterns for bf16 workloads, float32 otherwise.
    Rows at or beyond ``seq_lens[b]`` are zero.
    """
    seed = w.seed if seed is None else seed
    B, Hq, Hkv, dk, dv, r = w.batch, w.n_q_heads, w.n_kv_heads, w.d_k, w.d_v, w.rank
    G = w.group
    s_P, s_A, s_z, s_eps, s_V, s_qz, s_qn, s_ndl, s_len = np.random.SeedSequence(seed).spawn(9)
    gen = lambda s: np.random.Generator(np.random.PCG64(s))  # noqa: E731

    # orthonormal scoring basis per KV head
    gP = gen(s_P)
    P = np.empty((Hkv, dk, r), np.float32)
    for h in range(Hkv):
        Q, _ = np.linalg.qr(gP.standard_normal((dk, r)))
        P[h] = Q.astype(np.float32)

    gA = gen(s_A)
    A = gA.standard_normal((Hkv, dk, w.key_rank)) / np.sqrt(dk)  # fp64

    # sequence lengths
    if w.t_min is not None:
        seq_lens = gen(s_len).integers(w.t_min, w.t_max + 1, size=B).astype(np.int32)
    else:
        seq_lens = np.full(B, w.t_max, np.int32)
    if (seq_lens <= w.window).any():
        raise ValueError("every sequence must be longer than the window")

    # query
    qz = gen(s_qz).standard_normal((B, Hq, w.key_rank))
    qn = gen(s_qn).standard_normal((B, Hq, dk))
    q32 = np.empty((B, Hq, dk), np.float32)
    for hq in range(Hq):
        q32[:, hq] = (qz[:, hq] @ A[hq // G].T + 0.1 * qn[:, hq]).astype(np.float32)
    q = _store(w, q32)
    qv = _load(w, q)  # the values actually stored

    # bulk keys and values, chunked and seeded per (b, chunk)
    nchunks = (w.t_max + CHUNK - 1) // CHUNK
    z_seeds = s_z.spawn(B * nchunks)
    e_seeds = s_eps.spawn(B * nchunks)
    v_seeds = s_V.spawn(B * nchunks)
    k_cache = np.zeros((B, w.t_max, Hkv, dk), np.uint16 if w.dtype == "bf16" else np.float32)
    v_cache = None if w.mla else np.zeros((B, w.t_max, Hkv, dv), k_cache.dtype)
    A32 = A.astype(np.float32)

    def fill(job):
        b, c = job
        t0 = c * CHUNK
        t1 = min(int(seq_lens[b]), t0 + CHUNK)
        if t1 <= t0:
            return
        n = t1 - t0
        z = gen(z_seeds[b * nchunks + c]).standard_normal((n, Hkv, w.key_rank), dtype=np.float32)
        e = gen(e_seeds[b * nchunks + c]).standard_normal((n, Hkv, dk), dtype=np.float32)
        kk = np.matmul(z.transpose(1, 0, 2), A32.transpose(0, 2, 1)).transpose(1, 0, 2)
        e *= np.float32(0.1)
        e += kk
        k_cache[b, t0:t1] = _store(w, e)
        if v_cache is not None:
            vv = gen(v_seeds[b * nchunks + c]).standard_normal((n, Hkv, dv), dtype=np.float32)
            v_cache[b, t0:t1] = _store(w, vv)

    jobs = [(b, c) for b in range(B) for c in range(nchunks)]
    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, jobs))

    # planted needles: distinct candidate positions per (sequence, KV head)
    gN = gen(s_ndl)
    needles = np.zeros((B, Hkv, w.n_needles), np.int32)
    for b in range(B):
        n_cand = int(seq_lens[b]) - w.window
        m = min(w.n_needles, n_cand)
        for h in range(Hkv):
            pos = np.sort(gN.choice(n_cand, size=m, replace=False)).astype(np.int32)
            needles[b, h, :m] = pos
            for j in range(m):
                hq = (2 * j) % Hq if w.mla else h * G + (j % G)
                qq = qv[b, hq].astype(np.float64)
                row = (3.0 * qq / np.linalg.norm(qq)).astype(np.float32)
                k_cache[b, pos[j], h] = _store(w, row[None])[0]

    return {"workload": w, "P": P, "q": q, "k_cache": k_cache, "v_cache": v_cache,
            "seq_lens": seq_lens, "needles": needles}
