"""Shared helpers for the GPU parity tests: moving seeded inputs to the device,
descriptors from workloads, and the comparison rules (set tolerance, relative L2)."""
from __future__ import annotations

import numpy as np
import torch

import token_level_sparse_dim_amd as J
from oracle import jssa_oracle as O
from synth import Workload

DEV = "cuda"


def desc_for(w: Workload, reduce=J.REDUCE_MAX, out_dtype=J.F32, kp_dtype=None, **over) -> J.Desc:
    dt = J.F32 if w.dtype == "f32" else J.BF16
    d = dict(batch=w.batch, n_q_heads=w.n_q_heads, n_kv_heads=w.n_kv_heads, d_k=w.d_k, d_v=w.d_v,
             rank=w.rank, t_max=w.t_max, topk=w.topk, window=w.window, kv_dtype=dt,
             kp_dtype=dt if kp_dtype is None else kp_dtype, out_dtype=out_dtype, reduce=reduce,
             layout=J.LAYOUT_MLA if w.mla else J.LAYOUT_GQA, scale=w.scale)
    d.update(over)
    return J.Desc(**d)


def to_dev(x: np.ndarray) -> torch.Tensor:
    """numpy -> device tensor; uint16 arrays are bf16 bit patterns."""
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def to_host(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def kp_dtype_str(desc: J.Desc) -> str:
    return {J.BF16: "bf16", J.F32: "f32", J.FP8_E4M3: "fp8"}[desc.kp_dtype]


def oracle_kp(inp: dict, desc: J.Desc) -> np.ndarray:
    """The projected-key cache as the oracle stores it (the input both sides score)."""
    kp, _ = O.project_keys(inp["k_cache"], inp["P"], inp["seq_lens"], kp_dtype_str(desc))
    return kp


def rel_l2(a: np.ndarray, b: np.ndarray) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def check_sets_within_tolerance(idx_gpu, n_sel_gpu, s64, n_cand, seq_lens, topk, window, rel=1e-4):
    """End-to-end set rule: both sets have n_sel entries, the window parts are
    identical, and a token may be in only one of the two sets if its fp64 score
    lies within `rel` (relative) of the k-th score."""
    B, Hkv, _ = s64.shape
    ref_idx, ref_n = O.topk_select(s64, seq_lens, topk, window)
    worst = 0
    for b in range(B):
        for h in range(Hkv):
            n = int(ref_n[b, h])
            assert int(n_sel_gpu[b, h]) == n, (b, h, int(n_sel_gpu[b, h]), n)
            g = idx_gpu[b, h, :n]
            r = ref_idx[b, h, :n]
            assert (np.diff(g) > 0).all(), "indices must be strictly ascending"
            nc = int(n_cand[b])
            kk = min(topk, nc)
            assert np.array_equal(g[kk:], r[kk:]), "window differs"
            sg, sr = set(g[:kk].tolist()), set(r[:kk].tolist())
            diff = sg ^ sr
            if not diff:
                continue
            sk = O.kth_score(s64[b, h], nc, topk)
            # relative to |s_k|, floored at 1e-3 of the row's largest |score| for s_k near 0
            floor = rel * max(abs(sk), 1e-3 * float(np.nanmax(np.abs(s64[b, h, :nc]))))
            for t in diff:
                assert abs(s64[b, h, t] - sk) <= floor, (b, h, t, s64[b, h, t], sk)
            worst = max(worst, len(diff))
    return worst
