"""Plain, slow CPU oracle for token-level sparse decode attention (JSSA).

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run this module.  The
product path (the HIP library and its Python binding) never calls it, and it
shares no code, constants or helpers with that path.

Source of every definition: "Joint Subspace Sparse Attention for Efficient
Long-Context Decoding" (paperlayer.ai summary of arXiv 2610.19026v1), cited
below as *JSSA summary* with its section or figure.  Where the pages leave a
step open, the plainest reading is taken and named in the docstring
("Reading: ...").

Conventions
-----------
* All arithmetic is float64.  Inputs are float32 arrays, bf16 bit patterns
  stored as ``uint16`` or (projected keys only) FP8 E4M3 codes stored as
  ``uint8``; ``to_f64`` decodes all three exactly.
* Shapes: q ``[B, Hq, d_k]``; key/value cache ``[B, T_max, Hkv, d]``;
  basis ``P`` ``[Hkv, d_k, r]``; projected-key cache ``[B, Hkv, T_max, r]``;
  ``G = Hq // Hkv`` query heads per KV head, query head ``hq`` belongs to KV
  head ``hq // G``.
* A step for sequence ``b`` sees ``T_b = seq_lens[b]`` cached tokens.  The
  last ``W`` of them (``window``) are always attended; the scored candidates
  are ``t < T_b - W``.

Every function here is pinned by ``tests/test_oracle_pins.py`` against
something other than itself (closed forms, exact rational arithmetic,
brute-force enumeration, library routines, hand-derived golden values).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "to_f64", "round_to_bf16_bits", "e4m3_to_f64", "round_to_e4m3_bits", "project_keys", "project_query",
    "subspace_scores", "topk_select", "attention", "dense_attention", "decode",
    "n_selected", "kth_score", "gather_rows", "soft_vote",
]


# ---------------------------------------------------------------------------
# number formats
# ---------------------------------------------------------------------------
def to_f64(x: np.ndarray) -> np.ndarray:
    """Exact float64 value of a float32 array, of bf16 bit patterns (uint16)
    or of FP8 E4M3 codes (uint8)."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if x.dtype == np.uint8:
        return e4m3_to_f64(x)
    return x.astype(np.float64)


def e4m3_to_f64(code: np.ndarray) -> np.ndarray:
    """Value of FP8 E4M3 codes (the OCP 8-bit floating point format "E4M3",
    the FP8 of the projected scoring cache, JSSA summary Appendix A.3).

    Bit 7 is the sign, bits 6..3 the exponent field e (bias 7), bits 2..0 the
    mantissa m: e > 0 encodes (1 + m/8) * 2**(e-7), e == 0 encodes the
    subnormal m * 2**-9.  The all-ones pattern S.1111.111 is NaN; there are
    no infinities, so the largest magnitude is 1.75 * 2**8 = 448.
    """
    c = np.asarray(code, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.ldexp(1.0, e - 7))
    out = sign * mag
    return np.where((c & 0x7F) == 0x7F, np.nan, out)


def round_to_e4m3_bits(x: np.ndarray) -> np.ndarray:
    """Round exact values to FP8 E4M3, round-to-nearest, ties to even,
    saturating; return the codes (uint8).

    Reading: the pages store the scoring cache in FP8 without saying how
    values are rounded or whether a scale is applied; this takes the plainest
    scale-free encoding.  The spacing of representable values around |x| is
    2**(e-3) with e = floor(log2 |x|) clamped at the smallest normal exponent
    -6 (which covers the subnormals, spaced 2**-9); ``np.rint`` on x / spacing
    rounds half to even.  A result above the largest finite value saturates to
    +-448 (the format has no infinity); NaN becomes 0x7F.  -0.0 keeps its sign.
    """
    x = np.asarray(x, dtype=np.float64)
    fin = np.isfinite(x)
    ax = np.abs(np.where(fin, x, 0.0))
    nz = fin & (ax > 0)
    e = np.full(x.shape, -6, np.int64)
    e[nz] = np.maximum(np.floor(np.log2(ax[nz])).astype(np.int64), -6)
    lo = nz & (np.ldexp(1.0, e) > ax) & (e > -6)
    e[lo] -= 1
    hi = nz & (np.ldexp(1.0, e + 1) <= ax)
    e[hi] += 1
    spacing = np.ldexp(1.0, e - 3)
    mag = np.where(fin, np.rint(ax / spacing) * spacing, np.inf)
    mag = np.minimum(mag, 448.0)  # saturate (infinities included)
    # encode the magnitude: normal (1 + m/8) 2**k for mag >= 2**-6, else m 2**-9
    code = np.zeros(x.shape, np.int64)
    norm = mag >= 2.0 ** -6
    k = np.zeros(x.shape, np.int64)
    k[norm] = np.floor(np.log2(mag[norm])).astype(np.int64)
    k[norm & (np.ldexp(1.0, k) > mag)] -= 1
    k[norm & (np.ldexp(1.0, k + 1) <= mag)] += 1
    mant = np.where(norm, mag / np.ldexp(1.0, k) * 8.0 - 8.0, mag / 2.0 ** -9)
    code = np.where(norm, ((k + 7) << 3) | np.rint(mant).astype(np.int64), np.rint(mant).astype(np.int64))
    code = code | np.where(np.signbit(x), 0x80, 0)
    code = np.where(np.isnan(x), 0x7F, code)
    return code.astype(np.uint8)


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round exact values to bfloat16, round-to-nearest, ties to even; return bit patterns.

    bfloat16 keeps float32's 8-bit exponent and 8 significant bits (7 stored).
    The rounding is done once, from the float64 value: the spacing of
    representable values around |x| is 2**(e-7) with e = floor(log2 |x|)
    (clamped at the smallest normal exponent -126, which also covers the
    subnormals), and ``np.rint`` on x / spacing rounds half to even.  Values
    whose rounded magnitude reaches 2**128 overflow to infinity.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, np.float64)
    fin = np.isfinite(x)
    ax = np.abs(np.where(fin, x, 0.0))
    nz = fin & (ax > 0)
    e = np.full(x.shape, -126, np.int64)
    e[nz] = np.maximum(np.floor(np.log2(ax[nz])).astype(np.int64), -126)
    # log2 can be off by one next to powers of two: make 2**e <= |x| < 2**(e+1) exact
    lo = nz & (np.ldexp(1.0, e) > ax) & (e > -126)
    e[lo] -= 1
    hi = nz & (np.ldexp(1.0, e + 1) <= ax)
    e[hi] += 1
    spacing = np.ldexp(1.0, e - 7)
    out[fin] = np.rint(x[fin] / spacing[fin]) * spacing[fin]
    out[~fin] = x[~fin]
    out[fin & (np.abs(out) >= 2.0 ** 128)] = np.copysign(np.inf, x[fin & (np.abs(out) >= 2.0 ** 128)])
    f32 = out.astype(np.float32)  # exact: every bf16 value is a float32 value
    bits = (f32.view(np.uint32) >> 16).astype(np.uint16)
    bits[np.isnan(x)] = 0x7FC0
    return bits


# ---------------------------------------------------------------------------
# projected-key cache (the scoring-only cache)
# ---------------------------------------------------------------------------
def project_keys(k_cache: np.ndarray, P: np.ndarray, seq_lens: np.ndarray, out_dtype: str):
    """Projected-key cache ``Kp[b,h,t,:] = K[b,t,h,:] @ P[h]`` for t < T_b.

    JSSA summary §3.1 and §3.4: a scoring-only cache of keys projected onto
    the shared basis is kept per layer and KV head; §E.1: each newly generated
    key is projected into it at every step.  Appendix A.3 stores it in FP8
    (§E.2: FP8 halves the cache against BF16).  It is stored in the cache
    dtype ``out_dtype``, rounded once from the exact float64 product: 'bf16'
    (nearest even, uint16 bits), 'fp8' (E4M3 nearest even, saturating, uint8
    codes; ``round_to_e4m3_bits``) or 'f32' (float32 rounding).  Rows
    t >= T_b are zero.

    Returns ``(stored, exact)``: the stored cache and the float64 products,
    both ``[B, Hkv, T_max, r]``.
    """
    B, T, Hkv, _ = k_cache.shape
    r = P.shape[2]
    P64 = to_f64(P)
    exact = np.zeros((B, Hkv, T, r), np.float64)
    for b in range(B):
        n = int(seq_lens[b])
        for h in range(Hkv):
            exact[b, h, :n] = to_f64(k_cache[b, :n, h, :]) @ P64[h]
    if out_dtype == "bf16":
        stored = round_to_bf16_bits(exact)
    elif out_dtype == "fp8":
        stored = round_to_e4m3_bits(exact)
    elif out_dtype == "f32":
        stored = exact.astype(np.float32)
    else:
        raise ValueError(out_dtype)
    return stored, exact


def project_query(q: np.ndarray, P: np.ndarray, n_kv_heads: int) -> np.ndarray:
    """Projected query ``qp[b,hq,:] = q[b,hq,:] @ P[hq // G]`` (float64).

    JSSA summary §3.2: one orthonormal basis is applied to both queries and
    keys; query head hq uses the basis of the KV head it attends through.
    """
    B, Hq, _ = q.shape
    G = Hq // n_kv_heads
    q64, P64 = to_f64(q), to_f64(P)
    qp = np.empty((B, Hq, P.shape[2]), np.float64)
    for hq in range(Hq):
        qp[:, hq] = q64[:, hq] @ P64[hq // G]
    return qp


def subspace_scores(q, P, kp_cache, seq_lens, window: int, reduce: str = "max"):
    """Score every candidate token of every (sequence, KV head) in the subspace.

    JSSA summary Figure 1 and §3.1: each KV head scores its projected keys
    with the projected queries of its group of query heads.  The pages reduce
    the group by its *mean*; the build contract reduces it by the *max* over
    the group's heads.  Both are provided:

    * ``reduce='max'``:  s[b,h,t] = max_g  qp[b, hG+g] . Kp[b,h,t]
    * ``reduce='mean'``: s[b,h,t] = mean_g qp[b, hG+g] . Kp[b,h,t]
      (equal, by linearity, to scoring with the projected group-mean query).

    Reading: the stored projected keys (``kp_cache`` as given, decoded
    exactly) are what is scored; the float64 projection of the query is used.

    Returns ``s`` float64 ``[B, Hkv, T_max]``, defined for t < T_b - W and NaN
    elsewhere, and the candidate counts ``n_cand[b] = max(T_b - W, 0)``.
    """
    B, Hkv, T, _ = kp_cache.shape
    Hq = q.shape[1]
    G = Hq // Hkv
    qp = project_query(q, P, Hkv)
    s = np.full((B, Hkv, T), np.nan)
    n_cand = np.maximum(np.asarray(seq_lens, np.int64) - window, 0)
    for b in range(B):
        n = int(n_cand[b])
        for h in range(Hkv):
            per_head = to_f64(kp_cache[b, h, :n]) @ qp[b, h * G:(h + 1) * G].T  # [n, G]
            if reduce == "max":
                s[b, h, :n] = per_head.max(axis=1)
            elif reduce == "mean":
                s[b, h, :n] = per_head.mean(axis=1)
            else:
                raise ValueError(reduce)
    return s, n_cand


# ---------------------------------------------------------------------------
# selection
# ---------------------------------------------------------------------------
def n_selected(seq_len: int, topk: int, window: int) -> int:
    """Number of attended tokens: the window plus up to k scored candidates."""
    n_cand = max(seq_len - window, 0)
    return min(window, seq_len) + min(topk, n_cand)


def topk_select(scores: np.ndarray, seq_lens, topk: int, window: int):
    """Per-(sequence, KV head) token selection.

    JSSA summary Figure 1 and §1: each KV head keeps its own top-B positions
    (B is the budget, called k here), distinct across KV heads (§E.3,
    appendix A.3).  The build contract breaks ties towards the lower token
    index.  Reading for the hybrid case (appendix A.3 keeps local attention
    unchanged): the last W tokens are always attended and the top-k is taken
    from the rest.

    Ordering is a full stable sort: score descending, then index ascending.
    NaN scores rank below every number (and tie among themselves); -0.0 and
    +0.0 compare equal.  The output lists the selected candidates in
    ascending token order followed by the window ``T_b-W .. T_b-1``, padded
    with -1 to ``k + W``.

    Returns ``idx`` int32 ``[B, Hkv, k+W]`` and ``n_sel`` int32 ``[B, Hkv]``.
    """
    B, Hkv, _ = scores.shape
    idx = np.full((B, Hkv, topk + window), -1, np.int32)
    n_sel = np.zeros((B, Hkv), np.int32)
    for b in range(B):
        Tb = int(seq_lens[b])
        n_c = max(Tb - window, 0)
        win = np.arange(max(Tb - window, 0), Tb, dtype=np.int64)
        for h in range(Hkv):
            s = np.asarray(scores[b, h, :n_c], dtype=np.float64)
            t = np.arange(n_c)
            order = np.lexsort((t, -s))  # primary: -s ascending (NaN last); secondary: t
            chosen = np.sort(order[:min(topk, n_c)])
            sel = np.concatenate([chosen, win]).astype(np.int32)
            idx[b, h, :sel.size] = sel
            n_sel[b, h] = sel.size
    return idx, n_sel


def soft_vote(scores: np.ndarray, seq_lens, window: int, scale: float) -> np.ndarray:
    """Head-shared soft voting: one score per token of a sequence from all of
    its KV heads' scores.

    JSSA summary §E.3 compares per-KV-head selection (the method's default)
    with head-shared soft voting, which gives one token set per sequence; the
    pages do not spell the vote out.  Reading: each KV head votes with the
    softmax of its scaled scores over the sequence's candidates (t < T_b - W),
    and the votes are summed over the KV heads:

        vote[b, t] = sum_h exp(scale * s[b,h,t]) / sum_u exp(scale * s[b,h,u])

    (each head's votes sum to one).  NaN scores get no vote.  The shared set
    is ``topk_select`` of the vote (ties to the lower index), used by every
    KV head.  Returns ``vote`` float64 ``[B, 1, T_max]``, NaN past the
    candidates.
    """
    B, Hkv, T = scores.shape
    vote = np.full((B, 1, T), np.nan)
    for b in range(B):
        n = max(int(seq_lens[b]) - window, 0)
        if n == 0:
            continue
        acc = np.zeros(n)
        for h in range(Hkv):
            x = scale * np.asarray(scores[b, h, :n], dtype=np.float64)
            ok = ~np.isnan(x)
            if not ok.any():
                continue
            e = np.where(ok, np.exp(x - np.max(x[ok])), 0.0)
            acc += e / e.sum()
        vote[b, 0, :n] = acc
    return vote


def kth_score(scores: np.ndarray, n_cand: int, topk: int) -> float:
    """The k-th largest candidate score (the selection threshold), NaN-last order."""
    s = np.asarray(scores[:n_cand], np.float64)
    kk = min(topk, n_cand)
    order = np.lexsort((np.arange(n_cand), -s))
    return float(s[order[kk - 1]])


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------
def attention(q, k_cache, v_cache, idx, n_sel, scale: float):
    """Exact softmax attention of each query head over its KV head's selected tokens.

    JSSA summary Figure 1 and §3.1/§3.3: the query heads of a KV head share
    its selected positions and attend over the *original* full-dimensional
    keys and values (the projected cache is only for scoring).  Reading: the
    softmax is renormalised over the selected tokens only.

    ``v_cache`` may be a view of ``k_cache`` (MLA: the value is the first
    d_v columns of the shared latent row, §3.3).
    Returns ``out`` float64 ``[B, Hq, d_v]`` and the natural-log
    ``lse`` ``[B, Hq]`` = log sum_t exp(scale * q . K_t).
    """
    B, Hq, _ = q.shape
    Hkv = k_cache.shape[2]
    G = Hq // Hkv
    dv = v_cache.shape[3]
    q64 = to_f64(q)
    out = np.zeros((B, Hq, dv))
    lse = np.full((B, Hq), -np.inf)
    for b in range(B):
        for h in range(Hkv):
            rows = np.asarray(idx[b, h, :int(n_sel[b, h])], np.int64)
            if rows.size == 0:
                continue
            Kt = to_f64(k_cache[b, rows, h, :])
            Vt = to_f64(v_cache[b, rows, h, :])
            for g in range(G):
                hq = h * G + g
                logits = scale * (Kt @ q64[b, hq])
                m = logits.max()
                e = np.exp(logits - m)
                z = e.sum()
                out[b, hq] = (e @ Vt) / z
                lse[b, hq] = m + np.log(z)
    return out, lse


def dense_attention(q, k_cache, v_cache, seq_lens, scale: float):
    """Full-KV decode attention over every cached token t < T_b (the comparison path,
    JSSA summary §4.5)."""
    B, _, Hkv, _ = k_cache.shape
    kmax = int(np.max(seq_lens))
    idx = np.full((B, Hkv, kmax), -1, np.int32)
    n_sel = np.zeros((B, Hkv), np.int32)
    for b in range(B):
        Tb = int(seq_lens[b])
        idx[b, :, :Tb] = np.arange(Tb, dtype=np.int32)
        n_sel[b, :] = Tb
    return attention(q, k_cache, v_cache, idx, n_sel, scale)


def gather_rows(cache: np.ndarray, idx: np.ndarray, n_sel: np.ndarray) -> np.ndarray:
    """The gather of the gather-then-attend baseline: the selected rows copied,
    in list order, into a packed buffer ``[B, S, Hkv, d]`` (S = idx.shape[2]):
    ``packed[b, i, h] = cache[b, idx[b, h, i], h]`` for i < n_sel[b, h], zero
    past it.

    JSSA summary §2.2 and Figure 2(b): gathering the selected KV entries into
    a contiguous buffer before attention is the cost gather-free execution
    (§3.3) avoids; §4.7 compares the two on the same selected tokens.
    Attending densely over the first n_sel packed rows is the same attention
    as ``attention`` over the index list.
    """
    B, _, Hkv, d = cache.shape
    S = idx.shape[2]
    out = np.zeros((B, S, Hkv, d), dtype=cache.dtype)
    for b in range(B):
        for h in range(Hkv):
            n = int(n_sel[b, h])
            out[b, :n, h] = cache[b, idx[b, h, :n], h]
    return out


def decode(q, P, kp_cache, k_cache, v_cache, seq_lens, topk: int, window: int,
           scale: float, reduce: str = "max"):
    """One sparse decode step: subspace scores -> per-KV-head top-k -> attention.

    JSSA summary Figure 1 (scoring and execution path) and §E.1 (scan,
    selection, attention).  Returns a dict with ``scores``, ``n_cand``,
    ``idx``, ``n_sel``, ``out`` and ``lse``.
    """
    s, n_cand = subspace_scores(q, P, kp_cache, seq_lens, window, reduce)
    idx, n_sel = topk_select(s, seq_lens, topk, window)
    out, lse = attention(q, k_cache, v_cache, idx, n_sel, scale)
    return {"scores": s, "n_cand": n_cand, "idx": idx, "n_sel": n_sel, "out": out, "lse": lse}


def write_new_rows(cache: np.ndarray, new_rows: np.ndarray, pos) -> np.ndarray:
    """The step's new token rows written into a copy of a cache.

    JSSA summary §E.1 (each newly generated key and value is appended every
    step).  ``cache`` ``[B, T_max, H, d]``, ``new_rows`` ``[B, 1, H, d]``;
    ``cache[b, pos[b]] = new_rows[b, 0]`` for ``0 <= pos[b] < T_max``, other
    positions are left as they are.
    """
    out = np.array(cache, copy=True)
    for b in range(out.shape[0]):
        t = int(pos[b])
        if 0 <= t < out.shape[1]:
            out[b, t] = new_rows[b, 0]
    return out


def layer_stack_decode(layers, seq_lens, topk: int, window: int, scale: float,
                       indexer_every: int, reduce: str = "max"):
    """One decode step through a stack of layers that select only at indexer
    layers and reuse those lists in the layers after them.

    JSSA summary appendix C (with a model's own sparse-attention schedule,
    selection runs only at indexer layers and adjacent layers reuse the
    indices).  Reading: layer ``l`` is an indexer layer when
    ``l % indexer_every == 0``; it scores, selects and attends as
    :func:`decode`; every other layer attends over the most recent indexer
    layer's ``idx`` / ``n_sel`` with its own query and caches.  Every layer
    caches the same token positions.  ``layers``: dicts with ``q``,
    ``k_cache``, ``v_cache`` and, for indexer layers, ``P`` and
    ``kp_cache``.  Returns one dict per layer with ``out``, ``lse``, ``idx``,
    ``n_sel`` and ``indexer``.
    """
    res = []
    idx = n_sel = None
    for li, L in enumerate(layers):
        if li % indexer_every == 0:
            r = decode(L["q"], L["P"], L["kp_cache"], L["k_cache"], L["v_cache"], seq_lens,
                       topk, window, scale, reduce)
            idx, n_sel = r["idx"], r["n_sel"]
            res.append({"out": r["out"], "lse": r["lse"], "idx": idx, "n_sel": n_sel, "indexer": True})
        else:
            out, lse = attention(L["q"], L["k_cache"], L["v_cache"], idx, n_sel, scale)
            res.append({"out": out, "lse": lse, "idx": idx, "n_sel": n_sel, "indexer": False})
    return res
