"""Scalar pure-Python attention for tiny shapes (oracle pin; test infrastructure).

Two independent formulations used to pin the vectorised oracle:

* ``brute_sdpa``: the definition with ``math.fsum`` and ``math.exp`` over
  explicit loops, no numpy arithmetic;
* ``online_row``: one query row processed key by key with the running
  (max, denominator, output) state and the exp(old_max - new_max) rescale of
  the page "Agent 帮我写 CUDA：一个 Softmax Attention 算子的开发全记录",
  section 四 (Step 2), tiled-attention core idea. The page presents it as an
  exact rewriting of the softmax; the pin checks that claim against the
  definition.
"""
from __future__ import annotations

import math
from typing import List, Sequence


def _allowed(i: int, j: int, nq: int, nk: int, causal: bool, window: int) -> bool:
    delta = nk - nq
    if causal and j > i + delta:
        return False
    if window > 0 and j <= i + delta - window:
        return False
    return True


def brute_sdpa(q, k, v, *, scale: float, causal: bool = False, window: int = 0,
               softcap: float = 0.0, sink=None):
    """q [Hq][Nq][D], k/v [Hkv][Nk][D] nested lists -> (o [Hq][Nq][D], lse [Hq][Nq]).
    ``sink`` [Hq]: per-head sink logits, a valueless extra term of each row's
    normalisation (None: none)."""
    hq, hkv = len(q), len(k)
    group = hq // hkv
    nq, nk = len(q[0]), len(k[0])
    dv = len(v[0][0]) if nk else len(q[0][0])
    o = [[[0.0] * dv for _ in range(nq)] for _ in range(hq)]
    lse = [[-math.inf] * nq for _ in range(hq)]
    for h in range(hq):
        g = h // group
        for i in range(nq):
            scores = []
            for j in range(nk):
                if not _allowed(i, j, nq, nk, causal, window):
                    continue
                s = math.fsum(a * b for a, b in zip(q[h][i], k[g][j])) * scale
                if softcap > 0:
                    s = softcap * math.tanh(s / softcap)
                scores.append((j, s))
            if sink is not None:
                # the sink joins the normalisation as a valueless score (index -1)
                scores.append((-1, float(sink[h])))
            if not scores:
                continue
            m = max(s for _, s in scores)
            w = [(j, math.exp(s - m)) for j, s in scores]
            l = math.fsum(x for _, x in w)
            w = [(j, x) for j, x in w if j >= 0]
            for d in range(dv):
                o[h][i][d] = math.fsum(x * v[g][j][d] for j, x in w) / l
            lse[h][i] = m + math.log(l)
    return o, lse


def online_row(q_row: Sequence[float], keys: Sequence[Sequence[float]],
               values: Sequence[Sequence[float]], scale: float) -> List[float]:
    """The running-max recurrence over the keys of one row, one key at a time."""
    max_score = -math.inf
    denom = 0.0
    out = [0.0] * len(values[0])
    for kv, vv in zip(keys, values):
        score = math.fsum(a * b for a, b in zip(q_row, kv)) * scale
        old_max = max_score
        max_score = max(max_score, score)
        alpha = math.exp(old_max - max_score) if old_max != -math.inf else 0.0
        beta = math.exp(score - max_score)
        denom = denom * alpha + beta
        out = [o * alpha + beta * x for o, x in zip(out, vv)]
    return [o / denom for o in out]
