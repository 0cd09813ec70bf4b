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
    ``offset``: one causal offset, or a list with one per sequence.

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
    offs = list(offset) if isinstance(offset, (list, tuple)) else [offset] * B

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
                vis = [j for j in range(n_k) if _visible(i, j, lq[b], lk[b], causal, offs[b])]
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


def attention_tiny_packed(Q, K, V, GO, cu_q, cu_k, causal=False, offset=0):
    """The packed layout directly: Q[t][r][a] (rows t of all sequences one
    after another), K[t][g][a], V[t][g][l], GO[t][r][l]; sequence b owns rows
    cu_q[b] .. cu_q[b+1]-1 of Q/GO and cu_k[b] .. cu_k[b+1]-1 of K/V.  Row
    index i and key index j are counted from the sequence's first row.

    Returns O[t][r][l], lse[r][t], GQ[t][r][a], GK[t][g][a], GV[t][g][l]."""
    B = len(cu_q) - 1
    tq, tk = len(Q), len(K)
    H_q = len(Q[0]) if tq else (len(GO[0]) if GO else 0)
    H_kv = len(K[0]) if tk else 0
    d_h = len(Q[0][0]) if tq else (len(K[0][0]) if tk else 0)
    d_v = len(V[0][0]) if tk else 0
    grp = H_q // H_kv if H_kv else 1
    inv = 1.0 / math.sqrt(d_h) if d_h else 0.0
    offs = list(offset) if isinstance(offset, (list, tuple)) else [offset] * B
    O = [[[0.0] * d_v for _ in range(H_q)] for _ in range(tq)]
    lse = [[0.0] * tq for _ in range(H_q)]
    GQ = [[[0.0] * d_h for _ in range(H_q)] for _ in range(tq)]
    GK = [[[0.0] * d_h for _ in range(H_kv)] for _ in range(tk)]
    GV = [[[0.0] * d_v for _ in range(H_kv)] for _ in range(tk)]
    for b in range(B):
        q0, k0 = cu_q[b], cu_k[b]
        lq, lk = cu_q[b + 1] - q0, cu_k[b + 1] - k0
        for r in range(H_q):
            g = r // grp
            for i in range(lq):
                t = q0 + i
                vis = [j for j in range(lk) if (not causal) or j <= i + offs[b]]
                if not vis:
                    continue
                s = {j: sum(Q[t][r][a] * K[k0 + j][g][a] for a in range(d_h)) * inv for j in vis}
                m = max(s.values())
                e = {j: math.exp(s[j] - m) for j in vis}
                z = sum(e.values())
                p = {j: e[j] / z for j in vis}
                lse[r][t] = m + math.log(z)
                for l in range(d_v):
                    O[t][r][l] = sum(p[j] * V[k0 + j][g][l] for j in vis)
                ga = {j: sum(GO[t][r][l] * V[k0 + j][g][l] for l in range(d_v)) for j in vis}
                c = sum(p[j] * ga[j] for j in vis)
                gs = {j: p[j] * (ga[j] - c) for j in vis}
                for j in vis:
                    for l in range(d_v):
                        GV[k0 + j][g][l] += p[j] * GO[t][r][l]
                    for a in range(d_h):
                        GK[k0 + j][g][a] += gs[j] * Q[t][r][a] * inv
                for a in range(d_h):
                    GQ[t][r][a] = sum(gs[j] * K[k0 + j][g][a] for j in vis) * inv
    return {"O": O, "lse": lse, "GQ": GQ, "GK": GK, "GV": GV}
