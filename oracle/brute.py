"""Scalar-loop attention for tiny shapes (test infrastructure only).

A second, deliberately naive reading of the same definition as
`oracle.attention`: explicit loops over batch, head, query, key and dimension,
Python floats (binary64) and the math module only. It shares no helper with
`oracle.attention`, so the two agreeing pins the vectorised oracle's indexing,
head grouping, masks and log-sum-exp.

Definition (mslk flash_attn interface.py page, `_flash_attn_fwd`; the
visible-key rule is bottom-right aligned, inclusive at both window ends, with
causal meaning a right window of 0):
  key j is visible to query i of a (Sq, Sk) problem iff
    j >= i + (Sk - Sq) - window_left   (when window_left is bounded)
    j <= i + (Sk - Sq) + window_right  (when window_right is bounded)
"""
from __future__ import annotations

import math


def _visible(i, j, sq, sk, causal, wl, wr):
    diag = i + sk - sq
    right = 0 if causal else wr
    if wl is not None and wl >= 0 and j < diag - wl:
        return False
    if right is not None and right >= 0 and j > diag + right:
        return False
    return True


def attention_loops(q, k, v, scale, causal=False, window_left=None, window_right=None):
    """q[b][i][h][d], k[b][j][g][d], v[b][j][g][e] nested lists (or arrays).

    Returns (out[b][i][h][e], lse[b][h][i]) as nested Python lists.
    """
    B = len(q)
    Sq = len(q[0])
    Hq = len(q[0][0])
    D = len(q[0][0][0])
    Sk = len(k[0])
    Hkv = len(k[0][0])
    Dv = len(v[0][0][0])
    group = Hq // Hkv
    out = [[[[0.0] * Dv for _ in range(Hq)] for _ in range(Sq)] for _ in range(B)]
    lse = [[[0.0] * Sq for _ in range(Hq)] for _ in range(B)]
    for b in range(B):
        for h in range(Hq):
            g = h // group
            for i in range(Sq):
                scores = []
                for j in range(Sk):
                    if not _visible(i, j, Sq, Sk, causal, window_left, window_right):
                        continue
                    dot = 0.0
                    for d in range(D):
                        dot += float(q[b][i][h][d]) * float(k[b][j][g][d])
                    scores.append((j, scale * dot))
                if not scores:
                    lse[b][h][i] = -math.inf
                    continue
                mx = max(s for _, s in scores)
                total = 0.0
                for _, s in scores:
                    total += math.exp(s - mx)
                row_lse = mx + math.log(total)
                lse[b][h][i] = row_lse
                for e in range(Dv):
                    acc = 0.0
                    for j, s in scores:
                        acc += math.exp(s - row_lse) * float(v[b][j][g][e])
                    out[b][i][h][e] = acc
    return out, lse
