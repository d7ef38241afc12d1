"""Pure-Python brute force for tiny inputs: TEST INFRASTRUCTURE.

An independent second formulation of the same definition, used to pin the C
oracle.  It works on DENSE per-sequence keys and values (no pages, no block
table), expands KV heads by explicit repetition as boostr 0.2.0-beta.2
`expand_kv` does (repeat_interleave along the head axis), builds the explicit
additive 0 / -inf mask matrix of `build_attention_mask` (same page) on
absolute positions, and sums with math.fsum (exactly rounded sums).
"""
from __future__ import annotations

import math
from typing import List, Sequence, Tuple


def repeat_interleave_heads(rows: Sequence[Sequence[Sequence[float]]], repeats: int):
    """[L][Hkv][D] -> [L][Hkv*repeats][D], each head repeated `repeats` times in place."""
    return [[list(head) for head in token for _ in range(repeats)] for token in rows]


def mask_matrix(q_positions: Sequence[int], num_keys: int, causal: bool, window: int) -> List[List[float]]:
    """Additive mask on absolute positions: key j is hidden from a query at
    position p when (causal and j > p) or (window > 0 and j + window <= p)."""
    m = []
    for p in q_positions:
        row = []
        for j in range(num_keys):
            hidden = (causal and j > p) or (window > 0 and j + window <= p)
            row.append(-math.inf if hidden else 0.0)
        m.append(row)
    return m


def dense_attention(q: Sequence[Sequence[Sequence[float]]], k, v, q_positions: Sequence[int], hq: int,
                    hkv: int, scale: float, causal: bool, window: int
                    ) -> Tuple[List[List[List[float]]], List[List[float]]]:
    """q [n][hq][D]; k [L][hkv][D]; v [L][hkv][Dv] -> (out [n][hq][Dv], lse [n][hq])."""
    ke = repeat_interleave_heads(k, hq // hkv)
    ve = repeat_interleave_heads(v, hq // hkv)
    L = len(k)
    mask = mask_matrix(q_positions, L, causal, window)
    out, lse = [], []
    for i, qrow in enumerate(q):
        orow, lrow = [], []
        for h in range(hq):
            scores = [scale * math.fsum(a * b for a, b in zip(qrow[h], ke[j][h])) + mask[i][j]
                      for j in range(L)]
            m = max(scores) if scores else -math.inf
            if m == -math.inf:
                dv = len(v[0][0]) if L else 0
                orow.append([math.nan] * dv)
                lrow.append(-math.inf)
                continue
            w = [math.exp(s - m) if s != -math.inf else 0.0 for s in scores]
            total = math.fsum(w)
            dv = len(ve[0][h])
            orow.append([math.fsum(w[j] * ve[j][h][c] for j in range(L) if w[j] != 0.0) / total
                         for c in range(dv)])
            lrow.append(m + math.log(total))
        out.append(orow)
        lse.append(lrow)
    return out, lse
