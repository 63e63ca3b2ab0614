"""Brute-force softmax attention in pure Python (test infrastructure only).

For tiny shapes only (a few tokens, head_dim <= 8).  Uses ``math.fsum`` for
every sum so the result is as accurate as float64 allows, independent of
NumPy's summation order.  Same definition and layout as ``attention_fp64``.
"""

from __future__ import annotations

import math
from typing import List, Tuple


def brute_force_attention(q, k, v, scale: float) -> Tuple[list, list]:
    """``q``: nested lists ``[B][Sq][H][D]``; ``k``, ``v``: ``[B][Skv][H][D]``.

    Returns ``out[B][Sq][H][D]`` and ``lse[B][H][Sq]`` as nested lists.
    """
    B = len(q)
    Sq = len(q[0]) if B else 0
    H = len(q[0][0]) if Sq else len(k[0][0])
    D = len(q[0][0][0]) if Sq else len(k[0][0][0])
    Skv = len(k[0]) if B else 0
    out = [[[[0.0] * D for _ in range(H)] for _ in range(Sq)] for _ in range(B)]
    lse = [[[-math.inf] * Sq for _ in range(H)] for _ in range(B)]
    for b in range(B):
        for h in range(H):
            for i in range(Sq):
                if Skv == 0:
                    continue
                scores = []
                for j in range(Skv):
                    scores.append(scale * math.fsum(q[b][i][h][d] * k[b][j][h][d] for d in range(D)))
                m = max(scores)
                denom = math.fsum(math.exp(s - m) for s in scores)
                row_lse = m + math.log(denom)
                lse[b][h][i] = row_lse
                for d in range(D):
                    out[b][i][h][d] = math.fsum(math.exp(scores[j] - row_lse) * v[b][j][h][d]
                                                for j in range(Skv))
    return out, lse
