"""Softmax attention in float64, score matrix materialised (oracle; test infrastructure).

Steps, in the order the definition gives them (page "Agent 帮我写 CUDA：一个
Softmax Attention 算子的开发全记录", section 二, softmax(QK^T/sqrt(D))V; mask and
head-sharing readings as stated in this package's docstring):

1. S = (Q_h K_g^T) * scale for each query head h and its KV head g.
2. If softcap c > 0: S <- c * tanh(S / c).
3. Disallowed (i, j) become -inf.
4. m_i = max_j S_ij; P_ij = exp(S_ij - m_i); l_i = sum_j P_ij.
5. O_i = (sum_j P_ij V_j) / l_i; LSE_i = m_i + ln l_i.
   A row with no allowed key gives O_i = 0, LSE_i = -inf.

Attention sink (optional, one logit sigma_h per query head, natural-log units): a
score that takes part in every row's normalisation but carries no value, so step 4
takes m_i = max(max_j S_ij, sigma_h) and adds exp(sigma_h - m_i) to l_i. The
Ask-Don't-Equip page names "attention-sink" among the masks of the feature surface it
covers (section 研究动机) without defining it; this is the per-head sink logit of that
feature surface. A row with no allowed key then gives O_i = 0, LSE_i = sigma_h.

No blocking, fusion or reordering beyond what a library matmul does internally.
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np


def _allowed(nq: int, nk: int, *, causal: bool, window: int, q_pos: np.ndarray,
             nq_total: int, nk_valid: Optional[int] = None) -> Optional[np.ndarray]:
    """Boolean [Nq, Nk] mask, or None when every pair is allowed."""
    delta = nk - nq_total
    j = np.arange(nk)[None, :]
    i = q_pos[:, None]
    mask = None
    if causal:
        mask = j <= i + delta
    if window > 0:
        w = j > i + delta - window
        mask = w if mask is None else (mask & w)
    if nk_valid is not None and nk_valid < nk:
        v = np.broadcast_to(j < nk_valid, (nq, nk))
        mask = v if mask is None else (mask & v)
    return mask


def attention_probs(q: np.ndarray, k: np.ndarray, *, scale: float, causal: bool = False,
                    window: int = 0, softcap: float = 0.0) -> np.ndarray:
    """The normalised weights P [Hq, Nq, Nk] (tiny shapes only; for the pins)."""
    hq, nq, _ = q.shape
    hkv, nk, _ = k.shape
    group = hq // hkv
    mask = _allowed(nq, nk, causal=causal, window=window, q_pos=np.arange(nq), nq_total=nq)
    out = np.zeros((hq, nq, nk))
    for h in range(hq):
        s = (q[h] @ k[h // group].T) * scale
        if softcap > 0:
            s = softcap * np.tanh(s / softcap)
        if mask is not None:
            s = np.where(mask, s, -np.inf)
        m = s.max(axis=1)
        ok = np.isfinite(m)
        p = np.zeros_like(s)
        p[ok] = np.exp(s[ok] - m[ok, None])
        p[ok] /= p[ok].sum(axis=1, keepdims=True)
        out[h] = p
    return out


def sdpa_fp64(q: np.ndarray, k: np.ndarray, v: np.ndarray, *, scale: float, causal: bool = False,
              window: int = 0, softcap: float = 0.0, q_pos: Optional[np.ndarray] = None,
              nq_total: Optional[int] = None, sink: Optional[np.ndarray] = None
              ) -> Tuple[np.ndarray, np.ndarray]:
    """One sequence: q [Hq, Nq, D], k/v [Hkv, Nk, D] (float64) -> o [Hq, Nq, D], lse [Hq, Nq].

    ``q_pos`` gives the positions (0-based, within a query sequence of length
    ``nq_total``) of the supplied query rows, so that a sample of rows can be
    checked on its own; by default the rows are 0..Nq-1 of an Nq-row sequence.
    ``sink`` [Hq]: the per-head sink logits (None: no sink).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    hq, nq, d = q.shape
    hkv, nk, _ = k.shape
    if hq % hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    group = hq // hkv
    q_pos = np.arange(nq) if q_pos is None else np.asarray(q_pos, dtype=np.int64)
    nq_total = nq if nq_total is None else int(nq_total)
    mask = _allowed(nq, nk, causal=causal, window=window, q_pos=q_pos, nq_total=nq_total)
    o = np.zeros((hq, nq, v.shape[2]))
    lse = np.full((hq, nq), -np.inf)
    if sink is not None:
        sink = np.asarray(sink, dtype=np.float64)
        lse[:] = sink[:, None]  # the value of rows with no allowed key
    if nk == 0:
        return o, lse
    for h in range(hq):
        g = h // group
        s = (q[h] @ k[g].T) * scale
        if softcap > 0:
            s = softcap * np.tanh(s / softcap)
        if mask is not None:
            s = np.where(mask, s, -np.inf)
        if sink is not None:
            sg = float(sink[h])
            m = np.maximum(s.max(axis=1), sg)
            p = np.exp(s - m[:, None])
            l = p.sum(axis=1) + np.exp(sg - m)
            o[h] = (p @ v[g]) / l[:, None]
            lse[h] = m + np.log(l)
            continue
        m = s.max(axis=1)
        ok = np.isfinite(m)
        if not ok.all():
            s = s[ok]
            m = m[ok]
        p = np.exp(s - m[:, None])
        l = p.sum(axis=1)
        o[h, ok] = (p @ v[g]) / l[:, None]
        lse[h, ok] = m + np.log(l)
    return o, lse


def prefill_dense(q: np.ndarray, k: np.ndarray, v: np.ndarray, *, scale: float, causal: bool = False,
                  window: int = 0, softcap: float = 0.0, q_rows: Optional[np.ndarray] = None,
                  heads: Optional[np.ndarray] = None, sink: Optional[np.ndarray] = None):
    """Batched dense: q [B, Hq, Nq, D], k/v [B, Hkv, Nk, D] -> o [B, Hq', Nq', D], lse [B, Hq', Nq'].

    ``q_rows`` / ``heads`` restrict the output to a sample of query rows / query
    heads (the mask still uses each row's position in the full sequence).
    """
    b_, hq, nq, _ = q.shape
    hkv = k.shape[1]
    group = hq // hkv
    heads = np.arange(hq) if heads is None else np.asarray(heads)
    rows = np.arange(nq) if q_rows is None else np.asarray(q_rows)
    o = np.zeros((b_, len(heads), len(rows), v.shape[3]))
    lse = np.zeros((b_, len(heads), len(rows)))
    for b in range(b_):
        for n, h in enumerate(heads):
            g = h // group
            ob, lb = sdpa_fp64(q[b][h][rows][None], k[b][g][None], v[b][g][None], scale=scale,
                               causal=causal, window=window, softcap=softcap, q_pos=rows,
                               nq_total=nq, sink=None if sink is None else np.asarray(sink)[[h]])
            o[b, n] = ob[0]
            lse[b, n] = lb[0]
    return o, lse


def prefill_varlen(q: np.ndarray, k: np.ndarray, v: np.ndarray, cu_q: np.ndarray, cu_k: np.ndarray, *,
                   scale: float, causal: bool = True, window: int = 0, softcap: float = 0.0,
                   seqs: Optional[np.ndarray] = None, rows_per_seq: Optional[dict] = None,
                   heads: Optional[np.ndarray] = None, sink: Optional[np.ndarray] = None):
    """Ragged batch: q [T, Hq, D], k/v [Tk, Hkv, D] packed token-major by cu_seqlens.

    Sequences are independent; sequence b's queries attend to its own keys with
    the mask offset Nk_b - Nq_b. Returns (o [T, Hq, D], lse [Hq, T]) with rows
    outside the requested sample left as NaN.
    """
    hq = q.shape[1]
    heads = np.arange(hq) if heads is None else np.asarray(heads)
    o = np.full((q.shape[0], hq, v.shape[2]), np.nan)
    lse = np.full((hq, q.shape[0]), np.nan)
    seqs = range(len(cu_q) - 1) if seqs is None else seqs
    for b in seqs:
        q0, q1 = int(cu_q[b]), int(cu_q[b + 1])
        k0, k1 = int(cu_k[b]), int(cu_k[b + 1])
        rows = np.arange(q1 - q0)
        if rows_per_seq is not None and b in rows_per_seq:
            rows = np.asarray(rows_per_seq[b])
        qb = np.transpose(q[q0 + rows], (1, 0, 2))[heads]
        kb = np.transpose(k[k0:k1], (1, 0, 2))
        vb = np.transpose(v[k0:k1], (1, 0, 2))
        group = hq // k.shape[1]
        for n, h in enumerate(heads):
            g = h // group
            ob, lb = sdpa_fp64(qb[n:n + 1], kb[g:g + 1], vb[g:g + 1], scale=scale, causal=causal,
                               window=window, softcap=softcap, q_pos=rows, nq_total=q1 - q0,
                               sink=None if sink is None else np.asarray(sink)[[h]])
            o[q0 + rows, h] = ob[0]
            lse[h, q0 + rows] = lb[0]
    return o, lse


def gather_pages(cache: np.ndarray, block_table_row: np.ndarray, seq_len: int,
                 page_size: int = 16) -> np.ndarray:
    """Logical [L, Hkv, D] view of one sequence: token t sits in physical page
    block_table_row[t // page_size], slot t % page_size (integer work)."""
    t = np.arange(seq_len)
    pages = np.asarray(block_table_row)[t // page_size]
    return cache[pages, t % page_size]


def prefill_fp8(q_codes: np.ndarray, k_codes: np.ndarray, v_codes: np.ndarray, *, q_scale: float,
                k_scale: float, v_scale: float, scale: float, causal: bool = False, window: int = 0,
                softcap: float = 0.0, q_rows: Optional[np.ndarray] = None, heads: Optional[np.ndarray] = None,
                sink: Optional[np.ndarray] = None):
    """Dense prefill on fp8 (e4m3) inputs with per-tensor scales: the stored codes, already
    widened to their float64 values, times q_scale / k_scale / v_scale are the Q, K, V of
    the definition (fp8 inputs are a scenario axis of the Ask-Don't-Equip page, section
    研究动机; the per-tensor scale is the reading taken). Layout and sampling as
    prefill_dense.
    """
    return prefill_dense(np.asarray(q_codes) * float(q_scale), np.asarray(k_codes) * float(k_scale),
                         np.asarray(v_codes) * float(v_scale), scale=scale, causal=causal, window=window,
                         softcap=softcap, q_rows=q_rows, heads=heads, sink=sink)


def decode_paged(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray, block_table: np.ndarray,
                 seq_lens: np.ndarray, *, scale: float, k_scale: Optional[np.ndarray] = None,
                 v_scale: Optional[np.ndarray] = None, seqs: Optional[np.ndarray] = None,
                 page_size: int = 16, sink: Optional[np.ndarray] = None):
    """Single-token decode over a paged cache.

    q [S, Hq, D]; caches [P, page_size, Hkv, D] already widened to float64 (for
    fp8, the code values); k_scale / v_scale [Hkv] multiply the code values of
    KV head g. Sequence s's query attends to all of its seq_lens[s] cached keys.
    Returns (o [S', Hq, D], lse [S', Hq]) for the sequences in ``seqs``.
    """
    seqs = np.arange(q.shape[0]) if seqs is None else np.asarray(seqs)
    hq, d = q.shape[1], q.shape[2]
    o = np.zeros((len(seqs), hq, v_cache.shape[3]))
    lse = np.zeros((len(seqs), hq))
    for n, s in enumerate(seqs):
        L = int(seq_lens[s])
        kl = gather_pages(k_cache, block_table[s], L, page_size)  # [L, Hkv, D]
        vl = gather_pages(v_cache, block_table[s], L, page_size)
        if k_scale is not None:
            kl = kl * np.asarray(k_scale, dtype=np.float64)[None, :, None]
        if v_scale is not None:
            vl = vl * np.asarray(v_scale, dtype=np.float64)[None, :, None]
        ob, lb = sdpa_fp64(q[s][:, None, :], np.transpose(kl, (1, 0, 2)),
                           np.transpose(vl, (1, 0, 2)), scale=scale, sink=sink)
        o[n] = ob[:, 0]
        lse[n] = lb[:, 0]
    return o, lse


def prefill_paged(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray, block_table: np.ndarray,
                  cu_q: np.ndarray, seq_lens_k: np.ndarray, *, scale: float, causal: bool = True,
                  window: int = 0, softcap: float = 0.0, seqs: Optional[np.ndarray] = None,
                  rows_per_seq: Optional[dict] = None, heads: Optional[np.ndarray] = None,
                  page_size: int = 16, sink: Optional[np.ndarray] = None):
    """Chunked prefill over a paged cache: sequence b's queries q[cu_q[b]:cu_q[b+1]]
    ([T, Hq, D] packed) are its last Nq_b positions and attend to its Nk_b =
    seq_lens_k[b] keys, which sit in the cache pages its block-table row names
    (caches [P, page_size, Hkv, D], float64). The keys are gathered into one
    token-major array and the ragged definition above applies, with the mask offset
    Nk_b - Nq_b. Returns (o [T, Hq, D], lse [Hq, T]) (rows outside the sample NaN).
    """
    nseq = len(cu_q) - 1
    wanted = set(range(nseq)) if seqs is None else {int(b) for b in seqs}
    parts_k, parts_v, cu_k = [], [], [0]
    for b in range(nseq):
        # sequences outside the sample contribute no keys (their rows are not computed)
        L = int(seq_lens_k[b]) if b in wanted else 0
        parts_k.append(gather_pages(k_cache, block_table[b], L, page_size))
        parts_v.append(gather_pages(v_cache, block_table[b], L, page_size))
        cu_k.append(cu_k[-1] + L)
    k = np.concatenate(parts_k, axis=0)
    v = np.concatenate(parts_v, axis=0)
    return prefill_varlen(q, k, v, np.asarray(cu_q), np.asarray(cu_k), scale=scale, causal=causal,
                          window=window, softcap=softcap, seqs=seqs, rows_per_seq=rows_per_seq, heads=heads,
                          sink=sink)


def combine_partials(o_parts: np.ndarray, lse_parts: np.ndarray):
    """Merge results computed on disjoint key ranges (axis 0 indexes the ranges).

    With LSE_k the natural-log log-sum-exp of range k and O_k its normalised
    output: LSE = log sum_k exp(LSE_k) and O = sum_k exp(LSE_k - LSE) O_k.
    Ranges with LSE_k = -inf (no allowed key) carry zero weight.
    """
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    o_parts = np.asarray(o_parts, dtype=np.float64)
    m = lse_parts.max(axis=0)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    w = np.exp(lse_parts - m_safe[None])
    tot = w.sum(axis=0)
    with np.errstate(divide="ignore"):
        lse = np.where(tot > 0, m_safe + np.log(np.where(tot > 0, tot, 1.0)), -np.inf)
    coef = np.where(tot[None] > 0, w / np.where(tot > 0, tot, 1.0)[None], 0.0)
    o = (coef[..., None] * o_parts).sum(axis=0)
    return o, lse


def sdpa_backward_fp64(q: np.ndarray, k: np.ndarray, v: np.ndarray, do: np.ndarray, *, scale: float,
                       causal: bool = False, window: int = 0, softcap: float = 0.0,
                       sink: Optional[np.ndarray] = None):
    """Gradients of the forward definition for one sequence: q [Hq, Nq, D], k/v [Hkv, Nk, D],
    do = dL/dO [Hq, Nq, D] -> (dq, dk, dv) of the same shapes (float64).

    The backward pass is named by the Ask-Don't-Equip page (section 局限与改进: forward
    only, a backward pass as the next step) and not defined there; these are the
    derivatives of the definition, by the chain rule on its steps:
      S_raw = Q K^T, S = scale S_raw (or c tanh(scale S_raw / c)), P = softmax of the allowed
      S (with the sink in the normalisation when given), O = P V;
      dV = P^T dO; dP = dO V^T; dS = P * (dP - rowsum(dO * O));
      dS_raw = dS * scale (times 1 - tanh^2(scale S_raw / c) with a softcap);
      dQ = dS_raw K; dK = dS_raw^T Q. Query heads sharing a KV head add their dK, dV.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    hq, nq, _ = q.shape
    hkv, nk, _ = k.shape
    group = hq // hkv
    mask = _allowed(nq, nk, causal=causal, window=window, q_pos=np.arange(nq), nq_total=nq)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for h in range(hq):
        g = h // group
        s_raw = q[h] @ k[g].T
        if softcap > 0:
            t = np.tanh(s_raw * scale / softcap)
            s = softcap * t
        else:
            s = s_raw * scale
        if mask is not None:
            s = np.where(mask, s, -np.inf)
        m = s.max(axis=1)
        if sink is not None:
            m = np.maximum(m, float(sink[h]))
        ok = np.isfinite(m)
        p = np.zeros_like(s)
        p[ok] = np.exp(s[ok] - m[ok, None])
        l = p.sum(axis=1)
        if sink is not None:
            l = l + np.exp(float(sink[h]) - m)
        p[ok] /= l[ok, None]
        o = p @ v[g]
        dv[g] += p.T @ do[h]
        dp = do[h] @ v[g].T
        delta = (do[h] * o).sum(axis=1)
        ds = p * (dp - delta[:, None])
        ds_raw = ds * scale * ((1.0 - t * t) if softcap > 0 else 1.0)
        dq[h] = ds_raw @ k[g]
        dk[g] += ds_raw.T @ q[h]
    return dq, dk, dv


def prefill_backward_dense(q: np.ndarray, k: np.ndarray, v: np.ndarray, do: np.ndarray, *, scale: float,
                           causal: bool = False, window: int = 0, softcap: float = 0.0,
                           sink: Optional[np.ndarray] = None):
    """Batched dense: q/do [B, Hq, Nq, D], k/v [B, Hkv, Nk, D] -> (dq, dk, dv)."""
    out = [sdpa_backward_fp64(q[b], k[b], v[b], do[b], scale=scale, causal=causal, window=window,
                              softcap=softcap, sink=sink) for b in range(q.shape[0])]
    return tuple(np.stack([o[i] for o in out]) for i in range(3))
