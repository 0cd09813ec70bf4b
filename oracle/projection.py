"""float64 definition of the projections around the attention core.

TEST INFRASTRUCTURE ONLY (see the package docstring).

[A.10] "Appendix A.10 - Attention matrices and backpropagation", eq. A.10.10:
with row-major weights, Q = X W_Q, K = X W_K, V = X W_V for self-attention
(one input X feeds all three).  Eq. A.10.11: G_W = X^T G for each weight, and
the input's gradient is the SUM of its three branches,
    G_X = G_Q W_Q^T + G_K W_K^T + G_V W_V^T;
for cross-attention (query input X_q, key/value input X_kv) only the branches
that really share an input are summed: G_Xq = G_Q W_Q^T,
G_Xkv = G_K W_K^T + G_V W_V^T (same section).  [by-hand] "Working attention
out term by term", section three ends with the same three-branch sum and warns
that no branch may overwrite another.

Heads: the projected width H d of a row is split into H consecutive blocks of
d columns, head h owning columns h d .. h d + d - 1 (the concat order of
[A.10 sec. A.10.5], whose reshape/transpose changes only indexing).  The
weights of the three projections sit side by side in one matrix
W_qkv = [W_Q | W_K | W_V] of d_model rows and H_q d_h + H_kv d_h + H_kv d_v
columns (a storage choice; the products are the ones of eq. A.10.10).

Each product is a numpy matrix product (a library primitive); the branch sum
of eq. A.10.11 is written out as three products and two additions.
"""

from __future__ import annotations

import numpy as np

from .attention import InvalidArgument, attention_backward, attention_backward_packed


def split_qkv_weight(W_qkv, H_q: int, H_kv: int, d_h: int, d_v: int):
    """[W_Q | W_K | W_V] -> (W_Q, W_K, W_V)."""
    W = np.asarray(W_qkv, dtype=np.float64)
    a, b = H_q * d_h, H_q * d_h + H_kv * d_h
    if W.shape[1] != b + H_kv * d_v:
        raise InvalidArgument("W_qkv must have H_q d_h + H_kv d_h + H_kv d_v columns")
    return W[:, :a], W[:, a:b], W[:, b:]


def to_heads(Y, H: int, d: int) -> np.ndarray:
    """[B, n, H d] -> [B, H, n, d] (head h = columns h d .. h d + d - 1)."""
    B, n, _ = Y.shape
    return Y.reshape(B, n, H, d).transpose(0, 2, 1, 3)


def from_heads(Z) -> np.ndarray:
    """[B, H, n, d] -> [B, n, H d], the inverse of to_heads."""
    B, H, n, d = Z.shape
    return Z.transpose(0, 2, 1, 3).reshape(B, n, H * d)


def self_attention_backward(X, W_qkv, GO, *, H_q: int, H_kv: int, d_h: int, d_v: int, causal=False, offset=0,
                            seqlens_q=None, seqlens_k=None, cu_seqlens=None) -> dict:
    """Self-attention with its projections, forward and backward.

    X [B, n, d_model] (or [total rows, d_model] with cu_seqlens: packed
    sequences), W_qkv [d_model, C]; GO has the shape of O ([B, H_q, n, d_v],
    or [total, H_q, d_v] packed).  Returns Q, K, V (as heads), O, lse, their
    gradients GQ, GK, GV, and G_X (shape of X), G_W (shape of W_qkv)."""
    X = np.asarray(X, dtype=np.float64)
    W_Q, W_K, W_V = split_qkv_weight(W_qkv, H_q, H_kv, d_h, d_v)
    # eq. A.10.10
    PQ, PK, PV = X @ W_Q, X @ W_K, X @ W_V
    if cu_seqlens is None:
        if X.ndim != 3:
            raise InvalidArgument("X must be [B, n, d_model]")
        Q, K, V = to_heads(PQ, H_q, d_h), to_heads(PK, H_kv, d_h), to_heads(PV, H_kv, d_v)
        out = attention_backward(Q, K, V, GO, causal=causal, offset=offset, seqlens_q=seqlens_q,
                                 seqlens_k=seqlens_k)
        GPQ, GPK, GPV = from_heads(out["GQ"]), from_heads(out["GK"]), from_heads(out["GV"])
        Xr = X.reshape(-1, X.shape[-1])
        GPQ, GPK, GPV = (G.reshape(-1, G.shape[-1]) for G in (GPQ, GPK, GPV))
    else:
        if X.ndim != 2:
            raise InvalidArgument("packed X must be [total rows, d_model]")
        rows = X.shape[0]
        Q, K, V = PQ.reshape(rows, H_q, d_h), PK.reshape(rows, H_kv, d_h), PV.reshape(rows, H_kv, d_v)
        out = attention_backward_packed(Q, K, V, GO, cu_seqlens, cu_seqlens, causal=causal, offset=offset)
        GPQ, GPK, GPV = (out[g].reshape(rows, -1) for g in ("GQ", "GK", "GV"))
        Xr = X
    # eq. A.10.11: one weight gradient per branch, and the input's gradient
    # summed over its three branches
    G_WQ, G_WK, G_WV = Xr.T @ GPQ, Xr.T @ GPK, Xr.T @ GPV
    G_X = GPQ @ W_Q.T + GPK @ W_K.T + GPV @ W_V.T
    out = dict(out)
    out.update({"Q": Q, "K": K, "V": V, "G_X": G_X.reshape(X.shape),
                "G_W": np.concatenate([G_WQ, G_WK, G_WV], axis=1)})
    return out


def cross_attention_backward(Xq, Xkv, W_q, W_kv, GO, *, H_q: int, H_kv: int, d_h: int, d_v: int, causal=False,
                             offset=0, seqlens_q=None, seqlens_k=None) -> dict:
    """Cross-attention with its projections: Q = X_q W_Q, [K | V] = X_kv W_kv
    (W_kv = [W_K | W_V]).  Xq [B, n_q, d_q], Xkv [B, n_k, d_kv].  Returns O,
    lse, G_Xq = G_Q W_Q^T, G_Xkv = G_K W_K^T + G_V W_V^T (only the branches
    that share an input are summed), G_Wq, G_Wkv."""
    Xq = np.asarray(Xq, dtype=np.float64)
    Xkv = np.asarray(Xkv, dtype=np.float64)
    W_Q = np.asarray(W_q, dtype=np.float64)
    W_kv = np.asarray(W_kv, dtype=np.float64)
    if W_Q.shape[1] != H_q * d_h or W_kv.shape[1] != H_kv * (d_h + d_v):
        raise InvalidArgument("weight widths do not match the heads")
    W_K, W_V = W_kv[:, :H_kv * d_h], W_kv[:, H_kv * d_h:]
    Q = to_heads(Xq @ W_Q, H_q, d_h)
    K = to_heads(Xkv @ W_K, H_kv, d_h)
    V = to_heads(Xkv @ W_V, H_kv, d_v)
    out = attention_backward(Q, K, V, GO, causal=causal, offset=offset, seqlens_q=seqlens_q, seqlens_k=seqlens_k)
    GPQ = from_heads(out["GQ"]).reshape(-1, H_q * d_h)
    GPK = from_heads(out["GK"]).reshape(-1, H_kv * d_h)
    GPV = from_heads(out["GV"]).reshape(-1, H_kv * d_v)
    Xq2, Xkv2 = Xq.reshape(-1, Xq.shape[-1]), Xkv.reshape(-1, Xkv.shape[-1])
    G_Xq = GPQ @ W_Q.T
    G_Xkv = GPK @ W_K.T + GPV @ W_V.T
    out = dict(out)
    out.update({"Q": Q, "K": K, "V": V, "G_Xq": G_Xq.reshape(Xq.shape), "G_Xkv": G_Xkv.reshape(Xkv.shape),
                "G_Wq": Xq2.T @ GPQ, "G_Wkv": np.concatenate([Xkv2.T @ GPK, Xkv2.T @ GPV], axis=1)})
    return out
