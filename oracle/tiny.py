"""Second, independent oracle in pure Python (lists and the math module only).

TEST INFRASTRUCTURE ONLY.  Used by the tests to cross-check oracle.attention on
tiny shapes: it re-derives the same quantities element by element, with scalar
loops instead of numpy matrix products, so a transposed operand or a dropped
term in one of the two shows up as a disagreement.

Sources (see oracle/attention.py for the full page titles):
  scores and masked softmax   [A.10, eqs. A.10.1-A.10.3]
  G_V, G_A, G_S               [A.10, eqs. A.10.5-A.10.7]
  G_Q, G_K                    [A.10, eqs. A.10.8-A.10.9]
  grouped query heads         [A.10, sec. A.10.5]
The visible set of row i is { j < L_k[b] and (not causal or j <= i + offset) }
for rows i < L_q[b] (same reading as oracle.attention).
"""

from __future__ import annotations

import math


def _visible(i, j, lq, lk, causal, offset):
    if i >= lq or j >= lk:
        return False
    return (not causal) or j <= i + offset


def attention_tiny(Q, K, V, GO, causal=False, offset=0, seqlens_q=None, seqlens_k=None):
    """Q[b][r][i][a], K[b][g][j][a], V[b][g][j][l], GO[b][r][i][l] nested lists.

    Returns a dict of nested lists: O, lse, GQ, GK, GV, GS (per b, r)."""
    B = len(Q)
    H_q = len(Q[0]) if B else 0
    H_kv = len(K[0]) if B else 0
    n_q = len(Q[0][0]) if B else 0
    n_k = len(K[0][0]) if B else 0
    d_h = len(Q[0][0][0]) if (B and n_q) else (len(K[0][0][0]) if (B and n_k) else 0)
    d_v = len(V[0][0][0]) if (B and n_k) else 0
    grp = H_q // H_kv
    inv = 1.0 / math.sqrt(d_h)
    lq = seqlens_q if seqlens_q is not None else [n_q] * B
    lk = seqlens_k if seqlens_k is not None else [n_k] * B

    O = [[[[0.0] * d_v for _ in range(n_q)] for _ in range(H_q)] for _ in range(B)]
    lse = [[[0.0] * n_q for _ in range(H_q)] for _ in range(B)]
    GQ = [[[[0.0] * d_h for _ in range(n_q)] for _ in range(H_q)] for _ in range(B)]
    GK = [[[[0.0] * d_h for _ in range(n_k)] for _ in range(H_kv)] for _ in range(B)]
    GV = [[[[0.0] * d_v for _ in range(n_k)] for _ in range(H_kv)] for _ in range(B)]
    GSall = [[None] * H_q for _ in range(B)]

    for b in range(B):
        for r in range(H_q):
            g = r // grp
            q, k, v, go = Q[b][r], K[b][g], V[b][g], GO[b][r]
            GS = [[0.0] * n_k for _ in range(n_q)]
            for i in range(n_q):
                vis = [j for j in range(n_k) if _visible(i, j, lq[b], lk[b], causal, offset)]
                if not vis:
                    continue  # inactive padding row (active empty rows are rejected upstream)
                s = {}
                for j in vis:
                    acc = 0.0
                    for a in range(d_h):
                        acc += q[i][a] * k[j][a]
                    s[j] = acc * inv
                m = max(s[j] for j in vis)
                e = {j: math.exp(s[j] - m) for j in vis}
                z = sum(e[j] for j in vis)
                p = {j: e[j] / z for j in vis}
                lse[b][r][i] = m + math.log(z)
                for l in range(d_v):
                    O[b][r][i][l] = sum(p[j] * v[j][l] for j in vis)
                # backward of this row
                ga = {j: sum(go[i][l] * v[j][l] for l in range(d_v)) for j in vis}
                c = sum(p[j] * ga[j] for j in vis)
                for j in vis:
                    GS[i][j] = p[j] * (ga[j] - c)
                for j in vis:
                    for l in range(d_v):
                        GV[b][g][j][l] += p[j] * go[i][l]
                for a in range(d_h):
                    GQ[b][r][i][a] = sum(GS[i][j] * k[j][a] for j in vis) * inv
                for j in vis:
                    for a in range(d_h):
                        GK[b][g][j][a] += GS[i][j] * q[i][a] * inv
            GSall[b][r] = GS
    return {"O": O, "lse": lse, "GQ": GQ, "GK": GK, "GV": GV, "GS": GSall}
