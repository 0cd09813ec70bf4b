"""float64 definition of exact masked scaled dot-product attention (forward + backward).

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the benchmark's
CPU-baseline leg, never by the product path.

Sources (page titles as published; sections/equations named on each page):
  [A.10]     "Appendix A.10 - Attention matrices and backpropagation" (glenzli.com)
  [by-hand]  "Working attention out term by term" (aihero.club, attention-by-hand)
  [ch.15]    "Chapter 15: matrix formulas to look up" (math.zhuph.uk)
  [ch.31]    "Chapter 31: attention backpropagation and trainable retrieval"
             (eonloom AI-engineering handbook)

Everything is the plain definition, written out per (batch, query head) with
dense float64 numpy matrices.  No blocking, no online softmax, no fusion: a
reader can check each line against the equations named beside it.

Readings of points the pages leave open:
  * visible set of row i of sequence b:
        V_i = { j : j < L_k[b]  and  (not causal  or  j <= i + offset_b) }
    for active rows i < L_q[b]; 0-based indices.  The causal set {j <= i} is
    [A.10, sec. A.10.6]; the offset generalises the top-left rule of the
    [by-hand] exercise `causal_attention` (which defers offsets); padding
    removal is [A.10, sec. A.10.6].  offset_b is one value for the batch or
    one per sequence (each sequence's own cached history, [ch.31, sec. 1]).
  * packed layout: the sequences' rows stored one after another with no
    padding (row offsets cu_seqlens); sequence b is exactly the padded
    problem restricted to its own L_q[b] rows and L_k[b] keys.
  * rows i >= L_q[b] are inactive padding rows: O = 0, lse = 0, G_Q = 0 and
    they contribute nothing to G_K / G_V.
  * an ACTIVE row with an empty visible set is rejected ([A.10, sec. A.10.1]
    says softmax is undefined there; [ch.31, sec. 3] rejects such rows).
  * KV head of query head r: g(r) = floor(r / (H_q / H_kv)) (contiguous groups);
    [A.10, sec. A.10.5] names the map without a formula.
  * scale 1/sqrt(d_h) always (never d_v), [A.10, eq. A.10.1].
  * lse_i = m_i + ln(sum_{j in V_i} exp(S_ij - m_i)), natural log of the
    softmax denominator of the already-scaled scores.
"""

from __future__ import annotations

import math

import numpy as np


class OracleError(ValueError):
    """Base class of the oracle's input-rejection errors."""


class InvalidArgument(OracleError):
    """Inconsistent shapes, lengths or head grouping."""


class EmptyRow(OracleError):
    """An active query row has an empty visible set (softmax undefined)."""


# ----------------------------------------------------------------------------
# mask / grouping
# ----------------------------------------------------------------------------

def kv_group(r: int, H_q: int, H_kv: int) -> int:
    """KV head used by query head r: contiguous groups of H_q/H_kv query heads
    share one KV head ([A.10, sec. A.10.5]: MHA, MQA and GQA)."""
    return r // (H_q // H_kv)


def visible_mask(n_q: int, n_k: int, len_q: int, len_k: int,
                 causal: bool, offset: int) -> np.ndarray:
    """Boolean n_q x n_k matrix M with M[i, j] = (j in V_i) for active rows.

    Rows i >= len_q are inactive and all-False.  Keys j >= len_k are padding and
    never visible ([A.10, sec. A.10.6]).  With ``causal`` the row additionally
    sees only j <= i + offset ([A.10, sec. A.10.6] with offset 0; the offset is
    the chunked-query generalisation, [ch.31, sec. 1] new cached block against
    the full history)."""
    i = np.arange(n_q)[:, None]
    j = np.arange(n_k)[None, :]
    M = (i < len_q) & (j < len_k)
    if causal:
        M = M & (j <= i + offset)
    return M


def _lengths(lens, B: int, n: int, what: str) -> list[int]:
    if lens is None:
        return [n] * B
    lens = [int(x) for x in lens]
    if len(lens) != B:
        raise InvalidArgument(f"{what}: expected {B} lengths, got {len(lens)}")
    for x in lens:
        if x < 0 or x > n:
            raise InvalidArgument(f"{what}: length {x} outside [0, {n}]")
    return lens


def offsets_per_sequence(offset, B: int) -> list[int]:
    """The causal offset of every sequence: one int for all, or B values."""
    if np.ndim(offset) == 0:
        return [int(offset)] * B
    offs = [int(x) for x in offset]
    if len(offs) != B:
        raise InvalidArgument(f"offset: expected {B} per-sequence values, got {len(offs)}")
    return offs


def validate(B: int, H_q: int, H_kv: int, n_q: int, n_k: int,
             causal: bool, offset, seqlens_q=None, seqlens_k=None):
    """Resolve the per-sequence lengths and reject undefined problems.

    Returns (L_q, L_k) as lists.  Raises InvalidArgument for inconsistent
    grouping/lengths and EmptyRow when some active row would have an empty
    visible set ([A.10, sec. A.10.1]; [ch.31, sec. 3]).  The empty-row test
    is done by building each sequence's mask, not by a closed-form shortcut."""
    if B < 0 or n_q < 0 or n_k < 0 or H_q < 1 or H_kv < 1:
        raise InvalidArgument("negative size or no heads")
    if H_q % H_kv != 0:
        raise InvalidArgument("H_q must be a multiple of H_kv")
    L_q = _lengths(seqlens_q, B, n_q, "seqlens_q")
    L_k = _lengths(seqlens_k, B, n_k, "seqlens_k")
    offs = offsets_per_sequence(offset, B)
    for b in range(B):
        M = visible_mask(n_q, n_k, L_q[b], L_k[b], causal, offs[b])
        counts = M.sum(axis=1)
        if np.any(counts[: L_q[b]] == 0):
            raise EmptyRow(f"sequence {b}: an active query row sees no key")
    return L_q, L_k


# ----------------------------------------------------------------------------
# one (batch, query head): the definitions
# ----------------------------------------------------------------------------

def scores(q: np.ndarray, k: np.ndarray) -> np.ndarray:
    """S = Q K^T / sqrt(d_h)   ([A.10, eq. A.10.1]; [ch.31, sec. 1])."""
    return (q @ k.T) / math.sqrt(q.shape[1])


def masked_softmax(S: np.ndarray, M: np.ndarray):
    """Row softmax restricted to the visible set, with max subtraction.

    m_i = max_{j in V_i} S_ij, A_ij = exp(S_ij - m_i) / sum_{r in V_i} exp(S_ir - m_i)
    on V_i and 0 elsewhere ([A.10, eq. A.10.2]; the max shift leaves the result
    unchanged, [ch.15, sec. 15.1]).  Rows with no visible key (inactive rows)
    get A = 0, m = 0, ell = 0.  Returns (A, m, ell)."""
    active = M.any(axis=1)
    S_vis = np.where(M, S, -np.inf)
    m = np.where(active, S_vis.max(axis=1, initial=-np.inf), 0.0)
    E = np.where(M, np.exp(np.where(M, S, 0.0) - m[:, None]), 0.0)
    ell = E.sum(axis=1)
    A = np.zeros_like(S)
    A[active] = E[active] / ell[active, None]
    return A, m, ell


def score_grad(A: np.ndarray, GA: np.ndarray, M: np.ndarray):
    """G_S from G_A through the row softmax ([A.10, eq. A.10.7]; [ch.15, sec. 15.3];
    [ch.31, sec. 3]):  c_i = sum_{r in V_i} A_ir (G_A)_ir,
    (G_S)_ij = A_ij ((G_A)_ij - c_i) on V_i and 0 off V_i.  Returns (G_S, c)."""
    c = np.where(M, A * GA, 0.0).sum(axis=1)
    GS = np.where(M, A * (GA - c[:, None]), 0.0)
    return GS, c


def head_forward(q: np.ndarray, k: np.ndarray, v: np.ndarray, M: np.ndarray) -> dict:
    """Forward of one (batch, query head) on visible-set matrix M.

    Returns S, A, O = A V ([A.10, eq. A.10.3]) and lse (natural log of the
    softmax denominator of the scaled scores; 0 on inactive rows)."""
    S = scores(q, k)
    A, m, ell = masked_softmax(S, M)
    O = A @ v
    active = M.any(axis=1)
    lse = np.zeros(q.shape[0])
    lse[active] = m[active] + np.log(ell[active])
    return {"S": S, "A": A, "O": O, "lse": lse, "m": m, "ell": ell}


def head_backward(q, k, v, A, M, go) -> dict:
    """Backward of one (batch, query head) given upstream G_O.

    G_V = A^T G_O         [A.10, eq. A.10.5]
    G_A = G_O V^T         [A.10, eq. A.10.6]
    G_S                   [A.10, eq. A.10.7]  (score_grad)
    G_Q = G_S K / sqrt(d_h)    [A.10, eq. A.10.8]
    G_K = G_S^T Q / sqrt(d_h)  [A.10, eq. A.10.9]
    The returned G_K, G_V are this head's contributions; heads sharing a KV head
    are summed by the caller ([A.10, sec. A.10.5])."""
    d_h = q.shape[1]
    GV = A.T @ go
    GA = go @ v.T
    GS, c = score_grad(A, GA, M)
    GQ = (GS @ k) / math.sqrt(d_h)
    GK = (GS.T @ q) / math.sqrt(d_h)
    return {"GA": GA, "c": c, "GS": GS, "GQ": GQ, "GK": GK, "GV": GV}


# ----------------------------------------------------------------------------
# batched BHND tensors
# ----------------------------------------------------------------------------

def _shapes(Q, K, V):
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    if Q.ndim != 4 or K.ndim != 4 or V.ndim != 4:
        raise InvalidArgument("Q, K, V must be [B, H, n, d]")
    B, H_q, n_q, d_h = Q.shape
    Bk, H_kv, n_k, d_hk = K.shape
    Bv, H_kv2, n_k2, d_v = V.shape
    if Bk != B or Bv != B or H_kv2 != H_kv or n_k2 != n_k or d_hk != d_h:
        raise InvalidArgument("inconsistent Q/K/V shapes")
    return Q, K, V, (B, H_q, H_kv, n_q, n_k, d_h, d_v)


def attention_forward(Q, K, V, *, causal=False, offset=0,
                      seqlens_q=None, seqlens_k=None, keep=False) -> dict:
    """O [B,H_q,n_q,d_v] and lse [B,H_q,n_q] for the whole batch.

    With keep=True also returns the per-head S and A matrices (lists indexed by
    b*H_q + r) for inspection."""
    Q, K, V, (B, H_q, H_kv, n_q, n_k, d_h, d_v) = _shapes(Q, K, V)
    L_q, L_k = validate(B, H_q, H_kv, n_q, n_k, causal, offset, seqlens_q, seqlens_k)
    offs = offsets_per_sequence(offset, B)
    O = np.zeros((B, H_q, n_q, d_v))
    lse = np.zeros((B, H_q, n_q))
    kept = {"S": [], "A": [], "M": []}
    for b in range(B):
        M = visible_mask(n_q, n_k, L_q[b], L_k[b], causal, offs[b])
        for r in range(H_q):
            g = kv_group(r, H_q, H_kv)
            f = head_forward(Q[b, r], K[b, g], V[b, g], M)
            O[b, r] = f["O"]
            lse[b, r] = f["lse"]
            if keep:
                kept["S"].append(f["S"]); kept["A"].append(f["A"]); kept["M"].append(M)
    out = {"O": O, "lse": lse}
    if keep:
        out.update(kept)
    return out


def attention_backward(Q, K, V, GO, *, causal=False, offset=0,
                       seqlens_q=None, seqlens_k=None, keep=False) -> dict:
    """Forward and backward for the whole batch.

    Returns O, lse, G_Q, G_K, G_V, c (the row scalar of eq. A.10.7) and
    D = rowsum(G_O * O).  G_K/G_V of a KV head are the sums over the query
    heads r with g(r) = that head ([A.10, sec. A.10.5])."""
    Q, K, V, (B, H_q, H_kv, n_q, n_k, d_h, d_v) = _shapes(Q, K, V)
    GO = np.asarray(GO, dtype=np.float64)
    if GO.shape != (B, H_q, n_q, d_v):
        raise InvalidArgument("G_O must have the shape of O")
    L_q, L_k = validate(B, H_q, H_kv, n_q, n_k, causal, offset, seqlens_q, seqlens_k)
    offs = offsets_per_sequence(offset, B)
    O = np.zeros((B, H_q, n_q, d_v))
    lse = np.zeros((B, H_q, n_q))
    c = np.zeros((B, H_q, n_q))
    GQ = np.zeros_like(Q)
    GK = np.zeros_like(K)
    GV = np.zeros_like(V)
    kept = {"S": [], "A": [], "GS": [], "M": []}
    for b in range(B):
        M = visible_mask(n_q, n_k, L_q[b], L_k[b], causal, offs[b])
        for r in range(H_q):
            g = kv_group(r, H_q, H_kv)
            f = head_forward(Q[b, r], K[b, g], V[b, g], M)
            bw = head_backward(Q[b, r], K[b, g], V[b, g], f["A"], M, GO[b, r])
            O[b, r] = f["O"]
            lse[b, r] = f["lse"]
            c[b, r] = bw["c"]
            GQ[b, r] = bw["GQ"]
            GK[b, g] += bw["GK"]
            GV[b, g] += bw["GV"]
            if keep:
                kept["S"].append(f["S"]); kept["A"].append(f["A"])
                kept["GS"].append(bw["GS"]); kept["M"].append(M)
    D = (GO * O).sum(axis=-1)
    out = {"O": O, "lse": lse, "GQ": GQ, "GK": GK, "GV": GV, "c": c, "D": D}
    if keep:
        out.update(kept)
    return out


def attention_group(Q, K, V, GO, b: int, g: int, *, causal=False, offset=0,
                    seqlens_q=None, seqlens_k=None) -> dict:
    """Oracle restricted to one (sequence b, KV head g) and the query heads that
    share it: everything needed to check G_K[b, g] and G_V[b, g] exactly, and
    O / lse / G_Q for those query heads.  Used to sample full-size problems.

    Q/K/V/GO may be any array-likes indexable as [b, h] (e.g. numpy memmaps);
    only the slices of this group are read."""
    B, H_q, n_q, d_h = Q.shape
    _, H_kv, n_k, d_v = V.shape
    L_q, L_k = validate(B, H_q, H_kv, n_q, n_k, causal, offset, seqlens_q, seqlens_k)
    M = visible_mask(n_q, n_k, L_q[b], L_k[b], causal, offsets_per_sequence(offset, B)[b])
    heads = [r for r in range(H_q) if kv_group(r, H_q, H_kv) == g]
    k = np.asarray(K[b, g], dtype=np.float64)
    v = np.asarray(V[b, g], dtype=np.float64)
    out = {"heads": heads, "O": [], "lse": [], "GQ": [], "D": [],
           "GK": np.zeros((n_k, d_h)), "GV": np.zeros((n_k, d_v))}
    for r in heads:
        q = np.asarray(Q[b, r], dtype=np.float64)
        go = np.asarray(GO[b, r], dtype=np.float64) if GO is not None else None
        f = head_forward(q, k, v, M)
        out["O"].append(f["O"]); out["lse"].append(f["lse"])
        if go is not None:
            bw = head_backward(q, k, v, f["A"], M, go)
            out["GQ"].append(bw["GQ"])
            out["GK"] += bw["GK"]
            out["GV"] += bw["GV"]
            out["D"].append((go * f["O"]).sum(axis=1))
    for key in ("O", "lse", "GQ", "D"):
        out[key] = np.stack(out[key]) if out[key] else None
    return out


# ----------------------------------------------------------------------------
# packed ("varlen") layout
# ----------------------------------------------------------------------------

def _cu_lengths(cu, what: str) -> tuple[list[int], list[int]]:
    cu = [int(x) for x in cu]
    if len(cu) < 1 or cu[0] != 0:
        raise InvalidArgument(f"{what}: row offsets must start at 0")
    lens = [cu[i + 1] - cu[i] for i in range(len(cu) - 1)]
    if any(x < 0 for x in lens):
        raise InvalidArgument(f"{what}: row offsets must not decrease")
    return cu, lens


def attention_backward_packed(Q, K, V, GO, cu_seqlens_q, cu_seqlens_k, *, causal=False, offset=0) -> dict:
    """Forward and backward with the sequences packed one after another.

    Q [total_q, H_q, d_h], K [total_k, H_kv, d_h], V [total_k, H_kv, d_v],
    GO [total_q, H_q, d_v]; sequence b owns rows cu_seqlens_q[b] ..
    cu_seqlens_q[b+1]-1 of Q/GO and cu_seqlens_k[b] .. cu_seqlens_k[b+1]-1 of
    K/V.  Each sequence is computed on its own rows only (the padded
    definition above with B = 1 and n = its lengths, so no row of one
    sequence can reach another).  GO may be None (forward only).

    Returns O, GQ [total_q, H_q, .], GK, GV [total_k, H_kv, .], and lse, D
    [H_q, total_q]."""
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    cu_q, L_q = _cu_lengths(cu_seqlens_q, "cu_seqlens_q")
    cu_k, L_k = _cu_lengths(cu_seqlens_k, "cu_seqlens_k")
    B = len(L_q)
    if len(L_k) != B:
        raise InvalidArgument("cu_seqlens_q and cu_seqlens_k must describe the same sequences")
    if Q.shape[0] < cu_q[-1] or K.shape[0] < cu_k[-1] or V.shape[0] < cu_k[-1]:
        raise InvalidArgument("row offsets beyond the packed tensors")
    offs = offsets_per_sequence(offset, B)
    H_q, d_h = Q.shape[1], Q.shape[2]
    H_kv, d_v = V.shape[1], V.shape[2]
    O = np.zeros((Q.shape[0], H_q, d_v))
    GQ = np.zeros_like(Q)
    GK = np.zeros_like(K)
    GV = np.zeros_like(V)
    lse = np.zeros((H_q, Q.shape[0]))
    D = np.zeros((H_q, Q.shape[0]))
    for b in range(B):
        qs, ks = slice(cu_q[b], cu_q[b + 1]), slice(cu_k[b], cu_k[b + 1])
        # [rows, H, d] -> [1, H, rows, d]
        q = Q[qs].transpose(1, 0, 2)[None]
        k = K[ks].transpose(1, 0, 2)[None]
        v = V[ks].transpose(1, 0, 2)[None]
        if GO is None:
            f = attention_forward(q, k, v, causal=causal, offset=offs[b])
        else:
            go = np.asarray(GO, dtype=np.float64)[qs].transpose(1, 0, 2)[None]
            f = attention_backward(q, k, v, go, causal=causal, offset=offs[b])
            GQ[qs] = f["GQ"][0].transpose(1, 0, 2)
            GK[ks] = f["GK"][0].transpose(1, 0, 2)
            GV[ks] = f["GV"][0].transpose(1, 0, 2)
            D[:, qs] = f["D"][0]
        O[qs] = f["O"][0].transpose(1, 0, 2)
        lse[:, qs] = f["lse"][0]
    return {"O": O, "lse": lse, "GQ": GQ, "GK": GK, "GV": GV, "D": D}


# ----------------------------------------------------------------------------
# rotary position encoding (RoPE)
# ----------------------------------------------------------------------------

def rope_rotate(X, cos_sin, positions, inverse=False) -> np.ndarray:
    """Rotate each adjacent pair of columns (2k, 2k+1) of every row of X by the
    angle of that row's position: the 2-D block rotation of [ch.15, sec. 15.6]
    applied to q_i (or k_j), x~ = R(theta) x with
        x~_2k   = cos(theta) x_2k - sin(theta) x_2k+1
        x~_2k+1 = sin(theta) x_2k + cos(theta) x_2k+1,
    theta = theta(position, k) given by the table: cos_sin[pos, k] = (cos, sin).
    ``inverse`` applies R(theta)^T (the rotation by -theta): the backward of the
    rotation ([ch.31, sec. 5]: the transposed rotation of the upstream gradient).

    X: [..., n, d] with positions[n] the position of each row."""
    X = np.asarray(X, dtype=np.float64)
    cs = np.asarray(cos_sin, dtype=np.float64)
    pos = np.asarray(positions, dtype=np.int64)
    c = cs[pos, :, 0]   # [n, d/2]
    s = cs[pos, :, 1]
    if inverse:
        s = -s
    x0, x1 = X[..., 0::2], X[..., 1::2]
    Y = np.empty_like(X)
    Y[..., 0::2] = c * x0 - s * x1
    Y[..., 1::2] = s * x0 + c * x1
    return Y


def attention_backward_rope(Q, K, V, GO, cos_sin, *, causal=False, offset=0,
                            seqlens_q=None, seqlens_k=None) -> dict:
    """Attention with rotary positions on Q and K ([ch.15, sec. 15.6]): key j of
    a sequence sits at position j, query row i at position i + offset_b (its
    place in the key positions, the alignment the causal rule uses).  Forward
    on Q~ = R Q, K~ = R K; gradients G_Q = R^T G_Q~, G_K = R^T G_K~
    ([ch.31, sec. 5]); V is not rotated.  GO may be None (forward only)."""
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    B, H_q, n_q, _ = Q.shape
    n_k = K.shape[2]
    offs = offsets_per_sequence(offset, B)
    Qr = np.empty_like(Q)
    Kr = np.empty_like(K)
    for b in range(B):
        Qr[b] = rope_rotate(Q[b], cos_sin, np.arange(n_q) + offs[b])
        Kr[b] = rope_rotate(K[b], cos_sin, np.arange(n_k))
    kw = dict(causal=causal, offset=offset, seqlens_q=seqlens_q, seqlens_k=seqlens_k)
    if GO is None:
        return attention_forward(Qr, Kr, V, **kw)
    out = attention_backward(Qr, Kr, V, GO, **kw)
    for b in range(B):
        out["GQ"][b] = rope_rotate(out["GQ"][b], cos_sin, np.arange(n_q) + offs[b], inverse=True)
        out["GK"][b] = rope_rotate(out["GK"][b], cos_sin, np.arange(n_k), inverse=True)
    return out


def rope_table(n_pos: int, d_h: int, base: float = 10000.0) -> np.ndarray:
    """A cos/sin table [n_pos, d_h/2, 2] with the geometric frequencies
    omega_k = base^(-2k/d_h), theta = pos * omega_k (one common choice; the
    pages fix only that each 2-D block turns by position times a fixed
    frequency), rounded to float32 as the library receives it."""
    k = np.arange(d_h // 2)
    omega = base ** (-2.0 * k / d_h)
    theta = np.arange(n_pos)[:, None] * omega[None, :]
    return np.stack([np.cos(theta), np.sin(theta)], axis=-1).astype(np.float32)
